"""GPU parity of the prefill backward (dq, dk, dv, dg for dL/do = dO)
against the oracle's backward, through the C ABI.  The GPU forward
(scan + attention) provides hk, hv, o and lse, as in training.

Tolerances (max |err| over the whole tensor, relative to max |ref|; mean
|err| relative to mean |ref|): fp32 storage 1e-5 / 1e-5 (fp32 arithmetic,
other summation orders; observed about 1e-6); bf16 storage 3e-2 / 1e-2: every stored input of
the backward (q, k, v, g, dO, the states, o) carries a relative rounding of
up to 2^-8, P is formed in bf16 for the MFMAs, and the gate gradient uses
the stored bf16 state h_{t-1} where the oracle uses the exact one (with
h_{t-1} close to x_t the difference cancels, so elementwise relative errors
of dg are not bounded, only errors relative to the tensor's scale)."""
import zlib

import numpy as np
import pytest

import oracle
from dilated_sparse_attention_rat_amd import synth

from gpu_common import Checks, say, scale_of, to_dev, to_np

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

TOLB = {"f32": (1e-5, 1e-5), "bf16": (3e-2, 1e-2)}


def check_grad(name, got, ref, dtype):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - ref)
    mx = float(d.max()) / max(float(np.abs(ref).max()), 1e-30)
    mn = float(d.mean()) / max(float(np.abs(ref).mean()), 1e-30)
    say(f"  {name}: max|err|/max|ref|={mx:.2e}  mean|err|/mean|ref|={mn:.2e}  "
        f"(max|ref|={np.abs(ref).max():.3e})")
    tmax, tmean = TOLB[dtype]
    assert mx <= tmax, f"{name}: relative max error {mx}"
    assert mn <= tmean, f"{name}: relative mean error {mn}"


def gpu_forward_backward(inp, dO, D, W, dtype, bws=None, raw=False):
    """GPU forward, then the backward on `bws` (a fresh zero-filled
    workspace if None); the workspace's error word must stay 0."""
    import dilated_sparse_attention_rat_amd as rat
    q, k, v, g, do = (to_dev(a, dtype) for a in (inp["q"], inp["k"], inp["v"], inp["g"], dO))
    B, H, T, hd = q.shape
    st = q.dtype
    c = rat.alloc_cache(B, H, hd, T, D, W, st, "cuda")
    hk, hv = torch.empty_like(k), torch.empty_like(v)
    ws = rat.scan_workspace(B, H, T, hd, "cuda")
    rat.rat_scan_prefill(k, v, g, D, W, T, c["Kc"], c["Vc"], c["state_k"], c["state_v"], ws,
                         hk=hk, hv=hv, k_ring=c["k_ring"], v_ring=c["v_ring"])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    rat.rat_dilated_attn_prefill(q, hk, hv, c["Kc"], c["Vc"], D, W, T, o, lse)
    grads = [torch.full_like(q, float("nan")) for _ in range(4)]
    if bws is None:
        bws = rat.backward_workspace(B, H, T, hd, D, W, "cuda")
    rat.rat_prefill_backward(q, k, v, g, hk, hv, o, lse, do, D, W, *grads, bws)
    torch.cuda.synchronize()
    assert int(ws[2].item()) == 0, "a wait of the forward scan timed out"
    assert int(bws[2].item()) == 0, "a wait of the reverse scan timed out"
    if raw:
        return grads
    return dict(zip(("dq", "dk", "dv", "dg"), (to_np(x) for x in grads)))


CASES = [
    # label, B, H, T, hd, D, W, dtype
    ("bf16-hybrid-ragged", 2, 3, 700, 128, [4, 1, 16], [0, 37, 3], "bf16"),
    ("bf16-64-window", 1, 2, 333, 64, [3, 64], [0, 100], "bf16"),
    ("f32-128", 1, 2, 300, 128, [2, 7], [5, 0], "f32"),
    ("f32-64-window", 2, 2, 260, 64, [4, 9], [300, 1], "f32"),
    ("T1", 1, 2, 1, 128, [4, 1], [0, 3], "bf16"),
    ("D-beyond-T", 1, 2, 50, 64, [64, 100], [0, 0], "f32"),
    ("T129-dense", 1, 1, 129, 128, [1], [0], "bf16"),
    # windowless bf16 with at most 256 anchors per head: dq with resident anchors
    ("bf16-resident", 2, 3, 1000, 128, [4, 16, 8], [0, 0, 0], "bf16"),
    ("bf16-64-resident", 1, 2, 517, 64, [3, 5], [0, 0], "bf16"),
    ("resident-no-anchor", 1, 2, 40, 128, [64, 100], [0, 0], "bf16"),
    # reverse-scan trees of three and four levels (64-row chunks at bf16,
    # hd 128: 71 and 516 chunks; 32-row chunks at fp32: 79 chunks)
    ("bf16-tree-3-levels", 1, 2, 4500, 128, [16, 4], [0, 64], "bf16"),
    ("bf16-tree-4-levels", 1, 1, 33000, 128, [256], [0], "bf16"),
    ("f32-tree-3-levels", 1, 1, 2500, 128, [8], [16], "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    label, B, H, T, hd, D, W, dtype = case
    say(f"[backward] {label}: B={B} H={H} T={T} hd={hd} D={D} W={W} {dtype}")
    std = 1.0 if dtype == "f32" else hd ** -0.5
    seed = zlib.crc32(label.encode()) % 1000
    inp = synth.random_case(seed, B, H, T, hd, dtype, std, 3.0)
    dO = synth.random_case(seed + 1, B, H, T, hd, dtype, 1.0, 0.0)["q"]
    D, W = np.array(D, np.int32), np.array(W, np.int32)
    got = gpu_forward_backward(inp, dO, D, W, dtype)
    f = {n: inp[n].astype(np.float64) for n in "qkvg"}
    ref = oracle.backward(f["q"], f["k"], f["v"], f["g"], dO.astype(np.float64), D, W,
                          scale_of(hd), dtype == "bf16")
    chk = Checks()
    for n in ("dq", "dk", "dv", "dg"):
        chk(check_grad, n, got[n], ref[n], dtype)
    chk.done()


def test_backward_workload_size_sampled():
    """The 1.5B-like prefill shape (B=4, H=16, hd=128, T=4096, D=16): whole
    (b, h) slices of dq, dk, dv, dg against the oracle's backward of those
    slices (each slice is independent of the others)."""
    w = synth.WORKLOADS[1]
    say(f"[backward] workload 1 {w.name}: B={w.B} H={w.H} T={w.T}")
    inp = synth.prefill_inputs(w)
    dO = synth.random_case(4321, w.B, w.H, w.T, w.hd, w.dtype, 1.0, 0.0)["q"]
    D, W = np.array(w.D, np.int32), np.array(w.W, np.int32)
    got = gpu_forward_backward(inp, dO, D, W, w.dtype)
    chk = Checks()
    for (b, h) in [(0, 0), (w.B - 1, w.H - 1), (2, 7)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        f = {n: inp[n][sl].astype(np.float64) for n in "qkvg"}
        ref = oracle.backward(f["q"], f["k"], f["v"], f["g"], dO[sl].astype(np.float64),
                              D[h:h + 1], W[h:h + 1], w.scale, True)
        say(f" (b={b}, h={h})")
        for n in ("dq", "dk", "dv", "dg"):
            chk(check_grad, n, got[n][sl], ref[n], w.dtype)
    chk.done()


def test_backward_workspace_reused_bitwise():
    """One zero-filled workspace serves repeated calls and smaller calls: the
    reverse scan's chunk tree is tagged per launch, so the gradients equal,
    bit for bit, those computed on a fresh workspace (its composition order
    is fixed)."""
    import dilated_sparse_attention_rat_amd as rat
    B, H, hd, D, W = 2, 3, 128, np.array([4, 1, 16], np.int32), np.array([0, 37, 3], np.int32)
    big = synth.random_case(77, B, H, 1500, hd, "bf16", hd ** -0.5, 3.0)
    dO_big = synth.random_case(78, B, H, 1500, hd, "bf16", 1.0, 0.0)["q"]
    bws = rat.backward_workspace(B, H, 1500, hd, D, W, "cuda")
    say("[backward] one workspace: T=1500 twice, then T=700")
    first = gpu_forward_backward(big, dO_big, D, W, "bf16", bws=bws, raw=True)
    again = gpu_forward_backward(big, dO_big, D, W, "bf16", bws=bws, raw=True)
    for a, b in zip(first, again):
        assert torch.equal(a, b), "repeated call differs"
    small = {n: np.ascontiguousarray(big[n][:, :, :700]) for n in "qkvg"}
    dO_small = np.ascontiguousarray(dO_big[:, :, :700])
    reused = gpu_forward_backward(small, dO_small, D, W, "bf16", bws=bws, raw=True)
    fresh = gpu_forward_backward(small, dO_small, D, W, "bf16", raw=True)
    for a, b in zip(reused, fresh):
        assert torch.equal(a, b), "smaller call on a reused workspace differs"
