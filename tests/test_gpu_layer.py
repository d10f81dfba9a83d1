"""GPU parity of one RAT+ layer over a prefill (projections on the library's MFMA GEMM,
the gate fused into the scan, dilated attention, output projection) against
the oracle's layer, through the C ABI.

Tolerances, relative to the tensor's scale (max |err| / max |ref| and mean
|err| / mean |ref|): bf16 2e-2 for both -- the projections are rounded to
bf16 after an fp32 sum taken in another order than the oracle's float64 sum,
so single elements may land one bf16 step apart, and the recurrence and the
output projection carry that along (observed: about 4e-3 for out); fp32
1e-5 (observed: below 1e-6).  A stack of layers adds each layer's error to
the ones it is handed, so its bf16 bound on the max is 3e-2 (three layers of
about 4e-3 each, with margin); the mean keeps 2e-2.
"""
import zlib

import numpy as np
import pytest

import oracle

from gpu_common import Checks, say, to_dev, to_np

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

TOL = {"bf16": (2e-2, 2e-2), "f32": (1e-5, 1e-5)}


def check_rel(name, got, ref, dtype, tol=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - ref)
    mx = float(d.max()) / max(float(np.abs(ref).max()), 1e-30)
    mn = float(d.mean()) / max(float(np.abs(ref).mean()), 1e-30)
    say(f"  {name}: max|err|/max|ref|={mx:.2e}  mean|err|/mean|ref|={mn:.2e}")
    tmax, tmean = tol or TOL[dtype]
    assert mx <= tmax and mn <= tmean, f"{name}: {mx}, {mn}"


CASES = [
    # label, B, H, T, hd, dm, D, W, dtype
    ("bf16-hybrid", 2, 3, 300, 128, 256, [4, 1, 16], [0, 37, 3], "bf16"),
    ("bf16-64-resident", 1, 4, 640, 64, 192, [16, 8, 16, 32], [0, 0, 0, 0], "bf16"),
    ("f32-64", 2, 2, 130, 64, 96, [3, 5], [4, 0], "f32"),
    # d_model not a multiple of the GEMM's 32-wide K step: the input
    # projections take the register-staged GEMM (the output projection, K =
    # H*hd, the direct-to-LDS one); rows and columns past the tiles
    ("bf16-dm200-ragged", 1, 3, 333, 64, 200, [2, 7, 1], [0, 9, 0], "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_matches_oracle(case):
    import dilated_sparse_attention_rat_amd as rat
    label, B, H, T, hd, dm, D, W, dtype = case
    say(f"[layer] {label}: B={B} H={H} T={T} hd={hd} dm={dm} D={D} W={W} {dtype}")
    rng = np.random.default_rng(zlib.crc32(label.encode()) % 1000)
    HD = H * hd
    qkv_std = 1.0 if dtype == "f32" else hd ** -0.5

    def r(shape, std):
        a = (rng.standard_normal(shape) * std).astype(np.float32)
        return oracle.round_bf16(a).astype(np.float32) if dtype == "bf16" else a

    x = r((B, T, dm), 1.0)
    wq, wk, wv = (r((dm, HD), qkv_std / np.sqrt(dm)) for _ in range(3))
    wg = r((dm, HD), 1.0 / np.sqrt(dm))
    bg = np.full(HD, 3.0, np.float32)
    wo = r((HD, dm), 1.0 / np.sqrt(HD))
    D, W = np.array(D, np.int32), np.array(W, np.int32)
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda a: to_dev(a, dtype)
    cache = rat.alloc_cache(B, H, hd, T, D, W, st, "cuda")
    out = torch.empty((B, T, dm), dtype=st, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ws = rat.layer_workspace(rat.binding._dtype_code(out), B, H, T, hd, "cuda")
    bgt = torch.from_numpy(bg).cuda()
    for rep in range(2):  # the workspace is reused as is
        rat.rat_layer_prefill(dev(x), dev(wq), dev(wk), dev(wv), dev(wg), bgt, dev(wo), out, D, W,
                              H, hd, T, cache, ws, lse=lse)
        torch.cuda.synchronize()
        ref = oracle.layer_prefill(x, wq, wk, wv, wg, bg, wo, H, hd, D, W, hd ** -0.5,
                                   dtype == "bf16")
        chk = Checks()
        chk(check_rel, "out", to_np(out), ref["out"], dtype)
        chk(check_rel, "lse", to_np(lse), ref["lse"], dtype)
        chk(check_rel, "state_k", to_np(cache["state_k"]), ref["state_k"], dtype)
        chk(check_rel, "state_v", to_np(cache["state_v"]), ref["state_v"], dtype)
        assert int(ws[2].item()) == 0, "scan workspace reports a timed-out wait"
        chk.done()


def test_layer_workspace_reused_at_smaller_sizes():
    """One layer workspace, zeroed once, serves a call and then calls at a
    smaller T and a smaller B: the scan workspace heads it at a fixed
    offset, so its epoch and completion counters stay valid across sizes."""
    import dilated_sparse_attention_rat_amd as rat
    H, hd, dm = 3, 128, 256
    D, W = np.array([4, 1, 16], np.int32), np.array([0, 37, 3], np.int32)
    rng = np.random.default_rng(77)
    HD = H * hd

    def r(shape, std):
        return oracle.round_bf16((rng.standard_normal(shape) * std).astype(np.float32)).astype(np.float32)

    wq, wk, wv = (r((dm, HD), hd ** -0.5 / np.sqrt(dm)) for _ in range(3))
    wg = r((dm, HD), 1.0 / np.sqrt(dm))
    bg = np.full(HD, 3.0, np.float32)
    wo = r((HD, dm), 1.0 / np.sqrt(HD))
    dev = lambda a: to_dev(a, "bf16")
    ws = rat.layer_workspace(rat.binding._dtype_code(torch.empty(0, dtype=torch.bfloat16)), 2, H,
                             600, hd, "cuda")
    chk = Checks()
    for B, T in ((2, 600), (2, 257), (1, 600), (1, 90)):
        say(f"[layer] workspace reuse: B={B} T={T}")
        x = r((B, T, dm), 1.0)
        cache = rat.alloc_cache(B, H, hd, T, D, W, torch.bfloat16, "cuda")
        out = torch.empty((B, T, dm), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
        rat.rat_layer_prefill(dev(x), dev(wq), dev(wk), dev(wv), dev(wg),
                              torch.from_numpy(bg).cuda(), dev(wo), out, D, W, H, hd, T, cache, ws,
                              lse=lse)
        torch.cuda.synchronize()
        assert int(ws[2].item()) == 0, "scan workspace reports a timed-out wait"
        ref = oracle.layer_prefill(x, wq, wk, wv, wg, bg, wo, H, hd, D, W, hd ** -0.5, True)
        chk(check_rel, "out", to_np(out), ref["out"], "bf16")
        chk(check_rel, "lse", to_np(lse), ref["lse"], "bf16")
        chk(check_rel, "state_k", to_np(cache["state_k"]), ref["state_k"], "bf16")
        chk(check_rel, "state_v", to_np(cache["state_v"]), ref["state_v"], "bf16")
    chk.done()


def test_layer_workload_size_sampled():
    """The layer at the size the benchmark times (1.5B-like prefill, d_model =
    H*hd = 2048): the GPU runs all four batch rows, the oracle checks batch
    rows 0 and B-1 in full (output, lse, final states)."""
    import dilated_sparse_attention_rat_amd as rat
    from dilated_sparse_attention_rat_amd import synth
    w = synth.WORKLOADS[1]
    B, H, T, hd = w.B, w.H, w.T, w.hd
    dm = HD = H * hd
    say(f"[layer] workload 1 size: B={B} H={H} T={T} hd={hd} dm={dm}")
    rng = np.random.default_rng(1234)

    def r(shape, std):
        return oracle.round_bf16((rng.standard_normal(shape) * std).astype(np.float32)).astype(np.float32)

    x = r((B, T, dm), 1.0)
    wq, wk, wv = (r((dm, HD), w.qkv_std / np.sqrt(dm)) for _ in range(3))
    wg = r((dm, HD), 1.0 / np.sqrt(dm))
    bg = np.full(HD, float(w.g_bias), np.float32)
    wo = r((HD, dm), 1.0 / np.sqrt(HD))
    D, W = np.array(w.D, np.int32), np.array(w.W, np.int32)
    dev = lambda a: to_dev(a, "bf16")
    cache = rat.alloc_cache(B, H, hd, T, D, W, torch.bfloat16, "cuda")
    out = torch.empty((B, T, dm), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    ws = rat.layer_workspace(rat.binding._dtype_code(out), B, H, T, hd, "cuda")
    rat.rat_layer_prefill(dev(x), dev(wq), dev(wk), dev(wv), dev(wg), torch.from_numpy(bg).cuda(),
                          dev(wo), out, D, W, H, hd, T, cache, ws, lse=lse)
    torch.cuda.synchronize()
    chk = Checks()
    for b in (0, B - 1):
        say(f" batch row {b}")
        ref = oracle.layer_prefill(x[b:b + 1], wq, wk, wv, wg, bg, wo, H, hd, D, W, hd ** -0.5, True)
        chk(check_rel, "out", to_np(out[b:b + 1]), ref["out"], "bf16")
        chk(check_rel, "lse", to_np(lse[b:b + 1]), ref["lse"], "bf16")
        chk(check_rel, "state_k", to_np(cache["state_k"][b:b + 1]), ref["state_k"], "bf16")
        chk(check_rel, "state_v", to_np(cache["state_v"][b:b + 1]), ref["state_v"], "bf16")
    chk.done()


STACK = [
    # label, B, H, T, hd, dm, dtype, per layer (D, W)
    ("bf16-dense-dilated-hybrid", 2, 3, 300, 64, 192, "bf16",
     [([1, 1, 1], [0, 0, 0]), ([4, 4, 4], [0, 0, 0]), ([1, 8, 16], [0, 16, 5])]),
    ("f32-hybrid-dense", 1, 2, 150, 64, 96, "f32", [([8, 2], [3, 0]), ([1, 1], [0, 0])]),
    ("bf16-hd128-ragged", 1, 2, 333, 128, 200, "bf16", [([2, 7], [0, 9]), ([16, 1], [3, 0])]),
]


@pytest.mark.parametrize("case", STACK, ids=[c[0] for c in STACK])
def test_stack_matches_oracle(case):
    """A stack of layers, each with its own per-head dilation and window (the
    layer-wise hybrid), against the oracle's stack: the final output and
    every layer's final states, anchor cache and window ring.  A one-layer
    stack must equal the layer entry point bit for bit (same kernels)."""
    import dilated_sparse_attention_rat_amd as rat
    label, B, H, T, hd, dm, dtype, spec = case
    say(f"[stack] {label}: B={B} H={H} T={T} hd={hd} dm={dm} layers={spec} {dtype}")
    rng = np.random.default_rng(zlib.crc32(label.encode()) % 1000)
    HD = H * hd
    bf = dtype == "bf16"

    def r(shape, std):
        a = (rng.standard_normal(shape) * std).astype(np.float32)
        return oracle.round_bf16(a).astype(np.float32) if bf else a

    layers = []
    for D, W in spec:
        layers.append(dict(D=np.array(D, np.int32), W=np.array(W, np.int32),
                           w_q=r((dm, HD), 1 / np.sqrt(dm)), w_k=r((dm, HD), 1 / np.sqrt(dm)),
                           w_v=r((dm, HD), 1 / np.sqrt(dm)), w_g=r((dm, HD), 1 / np.sqrt(dm)),
                           b_g=np.full(HD, 1.0, np.float32), w_o=r((HD, dm), 2 / np.sqrt(HD))))
    x = r((B, T, dm), 1.0)
    st = torch.bfloat16 if bf else torch.float32
    dev = lambda a: to_dev(a, dtype)
    dl = [dict(D=ly["D"], W=ly["W"], w_q=dev(ly["w_q"]), w_k=dev(ly["w_k"]), w_v=dev(ly["w_v"]),
               w_g=dev(ly["w_g"]), b_g=torch.from_numpy(ly["b_g"]).cuda(), w_o=dev(ly["w_o"]))
          for ly in layers]
    caches = [rat.alloc_cache(B, H, hd, T, ly["D"], ly["W"], st, "cuda") for ly in layers]
    out = torch.empty((B, T, dm), dtype=st, device="cuda")
    code = rat.binding._dtype_code(out)
    ws = rat.stack_workspace(code, B, H, T, hd, dm, "cuda")
    xd = dev(x)
    tol = (3e-2, 2e-2) if bf else None
    ref = oracle.stack_prefill(x, layers, H, hd, hd ** -0.5, bf)
    for rep in range(2):  # the workspace is reused as is
        rat.rat_stack_prefill(xd, dl, out, H, hd, T, caches, ws)
        torch.cuda.synchronize()
        assert int(ws[2].item()) == 0, "scan workspace reports a timed-out wait"
        chk = Checks()
        chk(check_rel, "out", to_np(out), ref[-1]["out"], dtype, tol)
        for i, (c, rl) in enumerate(zip(caches, ref)):
            Kc, ring = oracle.build_cache(rl["hk"], layers[i]["D"], layers[i]["W"], T)
            Vc, vring = oracle.build_cache(rl["hv"], layers[i]["D"], layers[i]["W"], T)
            chk(check_rel, f"layer {i} state_k", to_np(c["state_k"]), rl["state_k"], dtype, tol)
            chk(check_rel, f"layer {i} state_v", to_np(c["state_v"]), rl["state_v"], dtype, tol)
            chk(check_rel, f"layer {i} Kc", to_np(c["Kc"]), Kc, dtype, tol)
            chk(check_rel, f"layer {i} Vc", to_np(c["Vc"]), Vc, dtype, tol)
            if ring is not None:
                chk(check_rel, f"layer {i} k_ring", to_np(c["k_ring"]), ring, dtype, tol)
                chk(check_rel, f"layer {i} v_ring", to_np(c["v_ring"]), vring, dtype, tol)
        chk.done()

    # one layer: the stack and the layer entry point run the same launches
    one = torch.empty_like(out)
    c1 = rat.alloc_cache(B, H, hd, T, layers[0]["D"], layers[0]["W"], st, "cuda")
    rat.rat_stack_prefill(xd, dl[:1], one, H, hd, T, [c1], ws)
    lw = rat.layer_workspace(code, B, H, T, hd, "cuda")
    two = torch.empty_like(out)
    c2 = rat.alloc_cache(B, H, hd, T, layers[0]["D"], layers[0]["W"], st, "cuda")
    L0 = dl[0]
    rat.rat_layer_prefill(xd, L0["w_q"], L0["w_k"], L0["w_v"], L0["w_g"], L0["b_g"], L0["w_o"], two,
                          L0["D"], L0["W"], H, hd, T, c2, lw)
    torch.cuda.synchronize()
    assert torch.equal(one, two), "one-layer stack differs from the layer entry point"
    assert torch.equal(c1["state_k"], c2["state_k"]) and torch.equal(c1["state_v"], c2["state_v"])
