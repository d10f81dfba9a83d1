"""Pins of the CPU oracle against facts fixed independently of it.

Each test ties one oracle function to something other than itself: a closed
form, a brute-force enumeration written here from the definition, an
independent formulation (associative scan, masked score matrix), a library
routine (torch scaled_dot_product_attention, torch bf16 conversion), or a
figure the pages state (the D-fold reduction of attention work and cache).
Planted-mistake tests at the end check that these pins would catch the
plausible errors.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _rand(shape, lo=None, hi=None):
    if lo is not None:
        return RNG.uniform(lo, hi, size=shape)
    return RNG.standard_normal(shape)


# --------------------------------------------------------------------------
# scan
# --------------------------------------------------------------------------
def _assoc_scan_hillis_steele(g, x):
    """Inclusive Hillis-Steele scan over the affine maps h -> a*h + b, with
    (a1,b1) then (a2,b2) = (a1*a2, a2*b1 + b2); returns b of each prefix."""
    a = g.copy()
    b = (1.0 - g) * x
    T = g.shape[2]
    step = 1
    while step < T:
        a_prev = np.concatenate([np.ones_like(a[:, :, :step]), a[:, :, :-step]], axis=2)
        b_prev = np.concatenate([np.zeros_like(b[:, :, :step]), b[:, :, :-step]], axis=2)
        b = a * b_prev + b
        a = a * a_prev
        step *= 2
    return b


def test_scan_equals_associative_scan():
    g = _rand((2, 3, 100, 5), 0.0, 1.0)
    x = _rand((2, 3, 100, 5))
    h, st = oracle.scan(g, x)
    ref = _assoc_scan_hillis_steele(g, x)
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(st, h[:, :, -1, :])


def test_scan_equals_unrolled_sum():
    """h_t = sum_s (1-g_s) x_s prod_{r=s+1..t} g_r (the recurrence unrolled)."""
    g = _rand((1, 1, 17, 3), 0.0, 1.0)
    x = _rand((1, 1, 17, 3))
    h, _ = oracle.scan(g, x)
    for t in range(17):
        acc = np.zeros(3)
        for s in range(t + 1):
            acc += (1 - g[0, 0, s]) * x[0, 0, s] * np.prod(g[0, 0, s + 1:t + 1], axis=0)
        np.testing.assert_allclose(h[0, 0, t], acc, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("gamma", [0.0, 0.3, 0.9, 0.999])
def test_scan_closed_form_step_response(gamma):
    T = 300
    g = np.full((1, 1, T, 2), gamma)
    x = np.ones((1, 1, T, 2))
    h, _ = oracle.scan(g, x)
    t = np.arange(T)
    np.testing.assert_allclose(h[0, 0, :, 0], 1.0 - gamma ** (t + 1), rtol=0, atol=1e-12)


def test_scan_closed_form_impulse():
    T, t0, gamma = 80, 13, 0.8
    g = np.full((1, 1, T, 1), gamma)
    x = np.zeros((1, 1, T, 1))
    x[0, 0, t0, 0] = 1.0
    h, _ = oracle.scan(g, x)
    t = np.arange(T)
    ref = np.where(t >= t0, (1 - gamma) * gamma ** np.maximum(t - t0, 0), 0.0)
    np.testing.assert_allclose(h[0, 0, :, 0], ref, rtol=1e-12, atol=1e-15)


def test_scan_gate_extremes():
    x = _rand((2, 2, 40, 4))
    h1, s1 = oracle.scan(np.ones_like(x), x)
    assert np.all(h1 == 0.0) and np.all(s1 == 0.0)
    h0, s0 = oracle.scan(np.zeros_like(x), x)
    np.testing.assert_array_equal(h0, x)  # bit-exact
    np.testing.assert_array_equal(s0, x[:, :, -1])


def test_scan_empty_sequence():
    g = np.zeros((1, 2, 0, 4))
    h, st = oracle.scan(g, g)
    assert h.shape == (1, 2, 0, 4)
    assert np.all(st == 0.0)


# --------------------------------------------------------------------------
# key set
# --------------------------------------------------------------------------
def _brute_keyset(t, D, W):
    """Key set of query t, written out from the definition as Python sets."""
    anchors = {j for j in range(t) if j % D == D - 1}
    window = set(range(max(0, t - W), t))
    return {t} | anchors | window


KEYSET_GRID = [(D, W) for D in [1, 2, 3, 4, 5, 6, 7, 8, 16, 64] for W in [0, 1, 3, 8, 64]]


@pytest.mark.parametrize("D,W", KEYSET_GRID)
def test_keyset_bruteforce(D, W):
    for t in range(64):
        ref = _brute_keyset(t, D, W)
        got = {j for j in range(t + 1) if oracle.in_keyset(t, j, D, W)}
        assert got == ref, (t, D, W)
        # nothing beyond t or below 0
        assert not oracle.in_keyset(t, t + 1, D, W)
        assert not oracle.in_keyset(t, -1, D, W)
        # cardinality closed form |S(t)| = 1 + min(W,t) + floor(max(0,t-W)/D)
        assert oracle.keyset_size(t, D, W) == 1 + min(W, t) + max(0, t - W) // D


@pytest.mark.parametrize("D,W", [(1, 0), (3, 0), (4, 2), (5, 7), (8, 0), (16, 3), (64, 64)])
def test_attention_keyset_readback(D, W):
    """With all keys equal the weights are uniform, and with one-hot values
    o_t[j] = 1/|S(t)| exactly on the key set: the set is read back from the
    attention function itself."""
    T = 64
    hd = 64
    q = _rand((1, 1, T, hd))
    hk = np.zeros((1, 1, T, hd))
    hv = np.eye(T)[None, None]  # hv[j] = e_j
    o, lse = oracle.attention(q, hk, hv, [D], [W], 0.125)
    for t in range(T):
        S = _brute_keyset(t, D, W)
        ref = np.zeros(hd)
        ref[list(S)] = 1.0 / len(S)
        np.testing.assert_allclose(o[0, 0, t], ref, rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[0, 0, t], math.log(len(S)), atol=1e-13)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _masked_softmax_attention(q, k, v, D, W, scale):
    """Independent formulation: full score matrix, boolean mask from the
    brute-force set, row softmax."""
    T = q.shape[0]
    mask = np.zeros((T, T), dtype=bool)
    for t in range(T):
        mask[t, list(_brute_keyset(t, D, W))] = True
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l, (m + np.log(l))[:, 0]


@pytest.mark.parametrize("D,W,T", [(1, 0, 50), (2, 0, 61), (4, 5, 64), (7, 3, 40), (16, 0, 64), (64, 10, 64)])
def test_attention_equals_masked_matrix_softmax(D, W, T):
    hd = 8
    q, k, v = _rand((1, 1, T, hd)), _rand((1, 1, T, hd)), _rand((1, 1, T, hd))
    o, lse = oracle.attention(q, k, v, [D], [W], 0.37)
    ref_o, ref_lse = _masked_softmax_attention(q[0, 0], k[0, 0], v[0, 0], D, W, 0.37)
    np.testing.assert_allclose(o[0, 0], ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], ref_lse, rtol=1e-12, atol=1e-12)


def _sdpa_causal(q, k, v, scale):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    return F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale).numpy()


def test_dense_case_equals_sdpa():
    """D = 1 without a window is dense causal attention (zhichai.net deep
    dive, section 2.2: D = 1 is the dense setting)."""
    B, H, T, hd = 2, 3, 70, 16
    q, k, v = _rand((B, H, T, hd)), _rand((B, H, T, hd)), _rand((B, H, T, hd))
    scale = 1 / math.sqrt(hd)
    o, _ = oracle.attention(q, k, v, [1] * H, [0] * H, scale)
    np.testing.assert_allclose(o, _sdpa_causal(q, k, v, scale), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("D", [2, 4, 16, 100])
def test_full_window_equals_sdpa(D):
    """A window of at least T-1 positions covers every earlier position."""
    B, H, T, hd = 1, 2, 45, 8
    q, k, v = _rand((B, H, T, hd)), _rand((B, H, T, hd)), _rand((B, H, T, hd))
    o, _ = oracle.attention(q, k, v, [D] * H, [T - 1] * H, 0.3)
    np.testing.assert_allclose(o, _sdpa_causal(q, k, v, 0.3), rtol=1e-10, atol=1e-12)


def test_constant_values_give_constant_output():
    B, H, T, hd = 1, 2, 64, 8
    q, k = _rand((B, H, T, hd)) * 5, _rand((B, H, T, hd)) * 5
    v = np.full((B, H, T, hd), 0.625)
    o, _ = oracle.attention(q, k, v, [4, 9], [0, 3], 1.0)
    np.testing.assert_allclose(o, 0.625, rtol=0, atol=1e-14)


def test_zero_gate_pipeline_is_plain_dilated_attention():
    """g = 0 makes the recurrent states equal to the raw keys and values."""
    B, H, T, hd = 1, 2, 64, 8
    q, k, v = _rand((B, H, T, hd)), _rand((B, H, T, hd)), _rand((B, H, T, hd))
    g = np.zeros_like(k)
    out = oracle.prefill(q, k, v, g, [4, 8], [0, 5], 0.35, st_bf16=False)
    o, _ = oracle.attention(q, k, v, [4, 8], [0, 5], 0.35)
    np.testing.assert_array_equal(out["o"], o)


def test_headwise_hybrid_equals_per_head_runs():
    """Per-head D/W in one call equals separate single-D calls per head
    (zhichai.net deep dive, section 六, head-wise hybrid)."""
    B, H, T, hd = 2, 4, 50, 8
    q, k, v = _rand((B, H, T, hd)), _rand((B, H, T, hd)), _rand((B, H, T, hd))
    D, W = [1, 1, 4, 4], [0, 0, 0, 6]
    o, lse = oracle.attention(q, k, v, D, W, 0.3)
    for h in range(H):
        oh, lh = oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], [D[h]], [W[h]], 0.3)
        np.testing.assert_array_equal(o[:, h:h + 1], oh)
        np.testing.assert_array_equal(lse[:, h:h + 1], lh)


def test_attention_rows_matches_full():
    B, H, T, hd = 2, 3, 90, 8
    q, k, v = _rand((B, H, T, hd)), _rand((B, H, T, hd)), _rand((B, H, T, hd))
    D, W = [3, 5, 1], [0, 4, 2]
    o, lse = oracle.attention(q, k, v, D, W, 0.3)
    rows = np.array([[0, 0, 0], [1, 2, 89], [0, 1, 45], [1, 0, 17]])
    orow, lrow = oracle.attention_rows(q, k, v, D, W, 0.3, rows)
    for r, (b, h, t) in enumerate(rows):
        np.testing.assert_array_equal(orow[r], o[b, h, t])
        np.testing.assert_array_equal(lrow[r], lse[b, h, t])


# --------------------------------------------------------------------------
# cache layout
# --------------------------------------------------------------------------
def test_anchor_offsets_and_cache_layout():
    B, H, T, hd = 2, 3, 37, 4
    D, W = [1, 4, 64], [0, 5, 3]
    T_cap = 50
    R, off = oracle.anchor_offsets(H, T_cap, D)
    assert R == 50 + 12 + 0
    assert list(off) == [0, 50, 62, 62]
    # position-coded states: channel 0 = t, 1 = h, 2 = b
    hs = np.zeros((B, H, T, hd))
    for b in range(B):
        for h in range(H):
            hs[b, h, :, 0] = np.arange(T)
            hs[b, h, :, 1] = h
            hs[b, h, :, 2] = b
    Kc, ring = oracle.build_cache(hs, D, W, T_cap)
    for b in range(B):
        for h in range(H):
            n = T // D[h]
            for a in range(R // 1):
                pass
            for a in range(n):
                row = Kc[b, off[h] + a]
                assert row[0] == a * D[h] + D[h] - 1 and row[1] == h and row[2] == b
            # rows past floor(T/D) stay untouched
            assert np.all(np.isnan(Kc[b, off[h] + n:off[h + 1]]))
            woff = sum(W[:h])
            for p in range(max(0, T - W[h]), T):
                row = ring[b, woff + p % W[h]]
                assert row[0] == p and row[1] == h and row[2] == b


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
@pytest.mark.parametrize("st_bf16", [False, True])
@pytest.mark.parametrize("D,W,T", [(4, 0, 40), (1, 0, 33), (8, 5, 64), (3, 100, 20), (16, 2, 0)])
def test_decode_equals_last_prefill_row(D, W, T, st_bf16):
    B, H, hd = 2, 2, 8
    q, k, v = _rand((B, H, T + 1, hd)), _rand((B, H, T + 1, hd)), _rand((B, H, T + 1, hd))
    g = _rand((B, H, T + 1, hd), 0.0, 1.0)
    full = oracle.prefill(q, k, v, g, [D] * H, [W] * H, 0.3, st_bf16)
    part = oracle.prefill(q[:, :, :T], k[:, :, :T], v[:, :, :T], g[:, :, :T], [D] * H, [W] * H, 0.3, st_bf16)
    o, sk, sv, hk1, hv1 = oracle.decode_step(
        q[:, :, T], k[:, :, T], v[:, :, T], g[:, :, T], part["state_k"], part["state_v"],
        part["hk"], part["hv"], [D] * H, [W] * H, 0.3, T, st_bf16)
    np.testing.assert_allclose(o, full["o"][:, :, T], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(sk, full["state_k"])
    np.testing.assert_array_equal(sv, full["state_v"])
    np.testing.assert_array_equal(hk1, full["hk"][:, :, T])
    np.testing.assert_array_equal(hv1, full["hv"][:, :, T])


# --------------------------------------------------------------------------
# bf16 storage rounding
# --------------------------------------------------------------------------
def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32),
        (RNG.standard_normal(2000) * 1e-30).astype(np.float32),
        (RNG.standard_normal(2000) * 1e30).astype(np.float32),
        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 2 ** -130]),
    ]).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x), ref)


# --------------------------------------------------------------------------
# the pages' own figure: D-fold cut of attention work and cache
# --------------------------------------------------------------------------
def test_pages_claim_dfold_reduction():
    """RAT+ abstract: dilation cuts attention FLOPs and the KV cache by D
    (64x at D = 64).  Check the exact counts of this definition against it."""
    with open(os.path.join(GOLDEN, "pages_claims.json")) as f:
        claims = json.load(f)
    for c in claims["dfold_reduction"]:
        T, D = c["T"], c["D"]
        total = sum(oracle.keyset_size(t, D, 0) for t in range(T))
        if T % D == 0:
            assert total == T * (T // D + 1) // 2
        dense = T * (T + 1) // 2
        ratio = dense / total
        assert abs(ratio - c["factor"]) / c["factor"] <= c["rel_tol"], (T, D, ratio)
        R, _ = oracle.anchor_offsets(1, T, [D])
        assert T / R == c["factor"]


# --------------------------------------------------------------------------
# planted mistakes: the pins above must catch them
# --------------------------------------------------------------------------
# --------------------------------------------------------------------------
# backward: gradient of a loss L with dL/do = dO
# --------------------------------------------------------------------------
def _bwd_case(B, H, T, hd, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, H, T, hd)) for _ in range(3))
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T, hd)) - 1.0))
    dO = rng.standard_normal((B, H, T, hd))
    return q, k, v, g, dO


BWD_FD_CASES = [
    # B, H, T, hd, D, W, scale, seed
    (1, 2, 40, 8, [3, 1], [0, 5], 0.35, 1),       # anchors, dense head, window
    (2, 1, 33, 4, [7], [2], 0.6, 2),              # sparse anchors + short window
    (1, 1, 10, 4, [16], [0], 0.5, 3),             # D > T: own position only
]


def _backward_fd(B, H, T, hd, D, W, scale, seed, n=8):
    """Central differences of the pinned forward (oracle.prefill) against
    oracle.backward at sampled elements of q, k, v and g; every sample set
    includes t = 0 (the longest reverse-recurrence chain)."""
    q, k, v, g, dO = _bwd_case(B, H, T, hd, seed)
    grads = oracle.backward(q, k, v, g, dO, D, W, scale, False)
    rng = np.random.default_rng(seed + 100)

    def loss(xs):
        return float((oracle.prefill(*xs, D, W, scale, False)["o"] * dO).sum())

    eps = 1e-6
    for i, name in enumerate(("q", "k", "v", "g")):
        idxs = [(0, 0, 0, 0)] + [tuple(int(rng.integers(0, s)) for s in (B, H, T, hd))
                                 for _ in range(n)]
        for idx in idxs:
            xs = [q.copy(), k.copy(), v.copy(), g.copy()]
            xs[i][idx] += eps
            lp = loss(xs)
            xs[i][idx] -= 2 * eps
            lm = loss(xs)
            fd = (lp - lm) / (2 * eps)
            an = grads["d" + name][idx]
            assert abs(fd - an) <= 1e-6 + 1e-5 * abs(fd), (name, idx, fd, an)


@pytest.mark.parametrize("case", BWD_FD_CASES)
def test_backward_matches_finite_differences(case):
    """The backward is the derivative of the forward: central differences of
    the oracle's own (separately pinned) prefill, loss sum(o * dO)."""
    _backward_fd(*case)


def test_backward_dense_zero_gate_equals_sdpa_autograd():
    """D = 1 with no window and g = 0 (states equal the inputs) is dense
    causal attention over k and v: gradients equal torch autograd of
    scaled_dot_product_attention (fp64, CPU); dg follows from the recurrence
    with h_{t-1} = x_{t-1}."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, H, T, hd = 1, 2, 37, 8
    q, k, v, _, dO = _bwd_case(B, H, T, hd, 9)
    g = np.zeros_like(q)
    scale = 0.4
    r = oracle.backward(q, k, v, g, dO, [1] * H, [0] * H, scale, False)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    o.backward(torch.from_numpy(dO))
    np.testing.assert_allclose(r["dq"], tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r["dk"], tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r["dv"], tv.grad.numpy(), rtol=1e-9, atol=1e-11)
    kp = np.concatenate([np.zeros_like(k[:, :, :1]), k[:, :, :-1]], axis=2)
    vp = np.concatenate([np.zeros_like(v[:, :, :1]), v[:, :, :-1]], axis=2)
    dg = tk.grad.numpy() * (kp - k) + tv.grad.numpy() * (vp - v)
    np.testing.assert_allclose(r["dg"], dg, rtol=1e-9, atol=1e-11)


def test_backward_storage_rounding_is_straight_through():
    """With g = 0 and inputs that are exact in bf16 the rounded states equal
    the exact ones, so the bf16-storage backward equals the exact one (the
    rounding enters the derivative as the identity)."""
    B, H, T, hd = 1, 2, 24, 8
    q, k, v, _, dO = _bwd_case(B, H, T, hd, 4)
    k, v = oracle.round_bf16(k), oracle.round_bf16(v)
    g = np.zeros_like(q)
    a = oracle.backward(q, k, v, g, dO, [3, 1], [2, 0], 0.3, True)
    b = oracle.backward(q, k, v, g, dO, [3, 1], [2, 0], 0.3, False)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])


# --------------------------------------------------------------------------
# layer: projections around the prefill
# --------------------------------------------------------------------------
def test_layer_identity_projections_reduce_to_prefill():
    """With W_q = W_k = W_v = W_o = I (dm = H*hd), W_g = 0 and a per-channel
    gate bias, the layer is the prefill of x split into heads with the gate
    sigmoid(b_g); per-head D and W make a head-layout mistake visible."""
    B, T, H, hd = 2, 30, 3, 4
    dm = H * hd
    x = _rand((B, T, dm))
    bg = _rand((H * hd,))
    eye, zero = np.eye(dm), np.zeros((dm, dm))
    D, W = [3, 1, 7], [0, 4, 2]
    r = oracle.layer_prefill(x, eye, eye, eye, zero, bg, eye, H, hd, D, W, 0.4, False)
    xh = x.reshape(B, T, H, hd).transpose(0, 2, 1, 3)
    g = np.broadcast_to(1.0 / (1.0 + np.exp(-bg.reshape(1, H, 1, hd))), xh.shape)
    ref = oracle.prefill(xh, xh, xh, g, D, W, 0.4, False)
    np.testing.assert_allclose(r["o"], ref["o"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["out"], ref["o"].transpose(0, 2, 1, 3).reshape(B, T, dm),
                               rtol=1e-12, atol=1e-14)


def test_layer_projections_bruteforce():
    """Every projection and the output projection, written as explicit sums
    over the model dimension for a tiny case."""
    B, T, H, hd, dm = 1, 6, 2, 4, 5
    x = _rand((B, T, dm))
    wq, wk, wv, wg = (_rand((dm, H * hd)) for _ in range(4))
    wo = _rand((H * hd, dm))
    bg = _rand((H * hd,))
    D, W = [2, 3], [1, 0]
    r = oracle.layer_prefill(x, wq, wk, wv, wg, bg, wo, H, hd, D, W, 0.5, False)

    def proj(w):
        y = np.zeros((B, H, T, hd))
        for b in range(B):
            for h in range(H):
                for t in range(T):
                    for c in range(hd):
                        y[b, h, t, c] = sum(x[b, t, j] * w[j, h * hd + c] for j in range(dm))
        return y

    q, k, v, gp = proj(wq), proj(wk), proj(wv), proj(wg)
    g = np.zeros_like(gp)
    for h in range(H):
        for c in range(hd):
            g[:, h, :, c] = 1.0 / (1.0 + math.e ** (-(gp[:, h, :, c] + bg[h * hd + c])))
    ref = oracle.prefill(q, k, v, g, D, W, 0.5, False)
    out = np.zeros((B, T, dm))
    for b in range(B):
        for t in range(T):
            for i in range(dm):
                out[b, t, i] = sum(ref["o"][b, h, t, c] * wo[h * hd + c, i]
                                   for h in range(H) for c in range(hd))
    np.testing.assert_allclose(r["out"], out, rtol=1e-10, atol=1e-12)



def _one_channel_layer(x, D, a, wo, scale, rnd):
    """Closed form of a layer with H = hd = d_model = 1, input projections
    q = k = v = a*x (rounded to the storage type, as stored) and a gate of
    exactly 0 (b_g = -1000: the recurrence then hands its input through),
    written from the definitions: the query at t attends to its own position
    and to the stride-D anchors j < t (j mod D = D-1), softmax with the given
    scale; out = o * wo with o as stored."""
    h = [rnd(a * v) for v in x]
    out = []
    for t in range(len(h)):
        keys = [j for j in range(t + 1) if j == t or j % D == D - 1]
        e = [math.exp(scale * h[t] * h[j]) for j in keys]
        o = sum(w * h[j] for w, j in zip(e, keys)) / sum(e)
        out.append(rnd(o) * wo)
    return out


@pytest.mark.parametrize("st_bf16", [False, True], ids=["f64", "bf16"])
def test_stack_two_layers_closed_form(st_bf16):
    """Two layers of different dilation (D = 1, then D = 2) over T = 5: the
    stack's output is the closed form of the second layer applied to the
    first one's output, rounded to the storage type in between.  Swapping
    the layers, or (bf16) handing the unrounded output over, gives another
    result, so a stack that runs its layers in the wrong order, skips one or
    hands over the wrong tensor fails."""
    def rnd(v):
        return float(oracle.round_bf16(np.array([v]))[0]) if st_bf16 else v

    x = [0.9, -1.3, 0.4, 2.1, -0.7]
    zero = np.zeros((1, 1))

    def layer(D, a, wo):
        w = np.full((1, 1), a)
        return dict(D=[D], W=[0], w_q=w, w_k=w, w_v=w, w_g=zero, b_g=np.array([-1000.0]),
                    w_o=np.full((1, 1), wo))

    scale = 0.8
    res = oracle.stack_prefill(np.array(x).reshape(1, 5, 1),
                               [layer(1, 1.0, 1.7), layer(2, 1.3, -0.6)], 1, 1, scale, st_bf16)
    mid = _one_channel_layer(x, 1, 1.0, 1.7, scale, rnd)
    ref = _one_channel_layer([rnd(v) for v in mid], 2, 1.3, -0.6, scale, rnd)
    np.testing.assert_allclose(res[0]["out"].ravel(), mid, rtol=1e-12, atol=0)
    np.testing.assert_allclose(res[1]["out"].ravel(), ref, rtol=1e-12, atol=0)
    swapped = _one_channel_layer(
        [rnd(v) for v in _one_channel_layer(x, 2, 1.3, -0.6, scale, rnd)], 1, 1.0, 1.7, scale, rnd)
    assert np.abs(np.array(swapped) - np.array(ref)).max() > 1e-3
    if st_bf16:
        unrounded = _one_channel_layer(mid, 2, 1.3, -0.6, scale, rnd)
        assert np.abs(np.array(unrounded) - np.array(ref)).max() > 1e-3


def test_stack_zero_output_projection_propagates_zeros():
    """A layer whose W_o is zero hands the next layer x = 0: its projections
    and states are then 0 and so is every later layer's output, whatever its
    weights; the first layer's own state is untouched by that."""
    B, T, H, hd, dm = 2, 20, 2, 4, 6
    HD = H * hd

    def layer(wo, D, W):
        return dict(D=D, W=W, w_q=_rand((dm, HD)), w_k=_rand((dm, HD)), w_v=_rand((dm, HD)),
                    w_g=_rand((dm, HD)), b_g=_rand((HD,)), w_o=wo)

    ls = [layer(np.zeros((HD, dm)), [3, 1], [2, 0]), layer(_rand((HD, dm)), [1, 5], [0, 3]),
          layer(_rand((HD, dm)), [2, 2], [1, 1])]
    x = _rand((B, T, dm))
    res = oracle.stack_prefill(x, ls, H, hd, 0.5, False)
    assert np.abs(res[0]["state_k"]).max() > 0
    for r in res:
        assert np.all(r["out"] == 0.0)
    for r in res[1:]:
        assert np.all(r["state_k"] == 0.0) and np.all(r["state_v"] == 0.0)

MUTANTS = [
    ("backward drops the softmax mean", "const double ds = p[j] * (dp[j] - delta);",
     "const double ds = p[j] * dp[j];", ["backward"]),
    ("reverse recurrence uses the current gate", "const double gn = (t + 1 < T) ? g[i + hd] : 0.0;",
     "const double gn = g[i];", ["backward"]),
    ("gate gradient sign", "dg[i] = lk * (pk - k[i]) + lv * (pv - v[i]);",
     "dg[i] = lk * (k[i] - pk) + lv * (v[i] - pv);", ["backward"]),
    ("input gradient misses 1-g", "dk[i] = (1.0 - g[i]) * lk;", "dk[i] = lk;", ["backward"]),
    # (description, original text, mutated text, pins expected to fail)
    ("anchor phase 0 instead of D-1", "if (j % D == D - 1) return 1;",
     "if (j % D == 0) return 1;", ["keyset", "readback"]),
    ("own position dropped", "if (j == t) return 1;", "if (0) return 1;",
     ["keyset", "readback"]),
    ("window off by one", "if (W > 0 && j >= t - W) return 1;",
     "if (W > 0 && j > t - W) return 1;", ["keyset", "readback"]),
    ("gate roles swapped", "s = g[i] * s + (1.0 - g[i]) * x[i];",
     "s = (1.0 - g[i]) * s + g[i] * x[i];", ["scan"]),
    ("state not reset per channel", "        double s = 0.0;\n        for (int t = 0; t < T; ++t) {",
     "        static double s = 0.0;\n        for (int t = 0; t < T; ++t) {", ["scan"]),
    ("softmax normaliser dropped", "    l += w;\n    for (int c = 0; c < hd; ++c) o[c] += w * hv[j * hd + c];",
     "    l += 1.0;\n    for (int c = 0; c < hd; ++c) o[c] += w * hv[j * hd + c];", ["softmax"]),
    ("scale applied twice", "    e *= scale;\n    double w = exp(e - m);",
     "    e *= scale * scale;\n    double w = exp(e - m);", ["softmax"]),
    ("transposed operand in the score", "for (int c = 0; c < hd; ++c) e += q[c] * hk[j * hd + c];\n    e *= scale;\n    double w",
     "for (int c = 0; c < hd; ++c) e += q[c] * hk[c * hd + j % hd];\n    e *= scale;\n    double w", ["softmax"]),
    ("bf16 rounding truncates", "double r = nearbyint(scaled);", "double r = trunc(scaled);", ["bf16"]),
    ("cache offset ignores earlier heads", "    if (off) off[h] = r;\n    r += T_cap / D[h];",
     "    if (off) off[h] = 0;\n    r += T_cap / D[h];", ["layout"]),
]

PIN_GROUPS = {
    "keyset": lambda: [test_keyset_bruteforce(D, W) for D, W in KEYSET_GRID],
    "readback": lambda: [test_attention_keyset_readback(D, W) for D, W in [(4, 2), (3, 0), (5, 7)]],
    "scan": lambda: (test_scan_equals_associative_scan(), test_scan_closed_form_impulse()),
    "softmax": lambda: [test_attention_equals_masked_matrix_softmax(D, W, T)
                        for D, W, T in [(2, 0, 61), (4, 5, 64)]],
    "bf16": test_round_bf16_matches_torch,
    "layout": test_anchor_offsets_and_cache_layout,
    "backward": lambda: [_backward_fd(*c, n=3) for c in BWD_FD_CASES[:2]],
}


@pytest.mark.parametrize("desc,orig,mut,groups", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, desc, orig, mut, groups):
    from oracle import oracle as orc
    src = orc.source_text()
    assert src.count(orig) == 1, desc
    path = orc.build_variant(src.replace(orig, mut), str(tmp_path / "mutant.so"))
    saved = orc._lib
    orc._lib = orc.load(path)
    try:
        for gname in groups:
            with pytest.raises(AssertionError):
                PIN_GROUPS[gname]()
    finally:
        orc._lib = saved
