"""Shared helpers of the GPU parity tests: run the HIP path through the
binding, and compare with the oracle at the stated tolerances.

Tolerances (applied to GPU output cast to fp64 against the fp64 oracle):
  fp32 storage: max |err| <= 1e-4;
  bf16 storage: max |err| <= 2e-2 and mean |err| <= 2e-3, plus a relative
  guard max |err| / max |ref| <= 2e-2 (the contract's absolute bound is loose
  against the ~3e-3 typical magnitude of o in these workloads);
  stored recurrent states (hk, hv, caches): within one storage ulp of the
  oracle's rounded state plus the fp32 rounding error of the recurrence
  (the fp32 state may sit on the other side of a rounding boundary; near a
  zero crossing the fp32 error, which is absolute at about 2^-24 times the
  state scale per step over the gate's memory 1/(1-g), exceeds one ulp of
  the tiny value): |err| <= ulp(ref) + 2^-16 * max|ref| over the checked
  slice; fp32 state: 1e-5 relative;
  cache layout / indices: bit-exact.
"""
import math
import sys

import numpy as np

import oracle

ULP_BF16 = 2.0 ** -7     # relative spacing of bf16 values, upper bound
TOL = {
    "f32": dict(max_abs=1e-4, mean_abs=1e-4, rel=1e-4),
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel=2e-2),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Checks:
    """Run every check of a test and report all failures at the end."""

    def __init__(self):
        self.fails = []

    def __call__(self, fn, *a, **k):
        try:
            fn(*a, **k)
        except AssertionError as e:
            self.fails.append(str(e))
            say(f"  FAIL: {e}")

    def done(self):
        assert not self.fails, "; ".join(self.fails)


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(torch_dtype(dtype))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_prefill(inp, D, W, T_cap, dtype, with_hk=True, fill=float("nan"), ws=None):
    """Run scan + attention on the GPU.  inp: dict of float32 arrays."""
    import torch
    import dilated_sparse_attention_rat_amd as rat
    q, k, v, g = (to_dev(inp[n], dtype) for n in "qkvg")
    B, H, T, hd = q.shape
    st = torch_dtype(dtype)
    cache = rat.alloc_cache(B, H, hd, T_cap, D, W, st, "cuda", fill=fill)
    hk = torch.full_like(k, fill) if with_hk else None
    hv = torch.full_like(v, fill) if with_hk else None
    if ws is None:
        ws = rat.scan_workspace(B, H, T, hd, "cuda")
    rat.rat_scan_prefill(k, v, g, D, W, T_cap, cache["Kc"], cache["Vc"], cache["state_k"],
                         cache["state_v"], ws, hk=hk, hv=hv, k_ring=cache["k_ring"],
                         v_ring=cache["v_ring"])
    out = dict(cache=cache, ws=ws, hk_t=hk, hv_t=hv, q_t=q)
    if with_hk:
        o = torch.full_like(q, fill)
        lse = torch.full((B, H, T), fill, dtype=torch.float32, device="cuda")
        rat.rat_dilated_attn_prefill(q, hk, hv, cache["Kc"], cache["Vc"], D, W, T_cap, o, lse)
        out.update(o_t=o, lse_t=lse)
    torch.cuda.synchronize()
    err = int(ws[2].item())  # workspace word 2: an aggregate wait timed out
    assert err == 0, "scan workspace reports a timed-out wait"
    return out


def check_float(name, got, ref, dtype, extra_rel=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    d = np.abs(got - ref)
    t = TOL[dtype]
    mx, mn = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 1.0
    rel = mx / max(scale, 1e-30)
    say(f"  {name}: max|err|={mx:.3e} mean|err|={mn:.3e} rel={rel:.3e} (max|ref|={scale:.3e})")
    assert mx <= t["max_abs"], f"{name}: max abs {mx} > {t['max_abs']}"
    assert mn <= t["mean_abs"], f"{name}: mean abs {mn} > {t['mean_abs']}"
    assert rel <= (extra_rel if extra_rel is not None else t["rel"]), f"{name}: rel {rel}"


def check_state_ulp(name, got, ref_rounded, dtype):
    """Stored states: within one storage ulp of the oracle's rounded state."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref_rounded, dtype=np.float64)
    d = np.abs(got - ref)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if dtype == "bf16":
        one_ulp = ULP_BF16 * np.abs(ref) + 1e-37
        lim = one_ulp + 2.0 ** -16 * scale
    else:
        one_ulp = 1e-5 * np.abs(ref) + 1e-6
        lim = one_ulp
    bad = d > lim
    say(f"  {name}: max|err|={d.max() if d.size else 0:.3e}, "
        f"{int((d > 0).sum())} of {d.size} differ, {int((d > one_ulp).sum())} beyond one ulp, "
        f"{int(bad.sum())} beyond the bound")
    if bad.any() or (d > one_ulp).any():
        idx = np.argsort((d - one_ulp).ravel())[-4:]
        for i in idx:
            say(f"    got={got.ravel()[i]:.9e} ref={ref.ravel()[i]:.9e} "
                f"err={d.ravel()[i]:.3e} ulp-bound={one_ulp.ravel()[i]:.3e}")
    assert not bad.any(), f"{name}: {int(bad.sum())} values beyond the bound"


def check_fp32_state(name, got, ref):
    d = np.abs(np.asarray(got, np.float64) - ref)
    lim = 1e-5 * np.abs(ref) + 1e-6
    say(f"  {name}: max|err|={d.max():.3e}")
    assert np.all(d <= lim), name


def oracle_prefill(inp, D, W, scale, dtype, rows=None, bh=None):
    """Oracle on the full input (rows=None) or on the (b, h) pairs in bh with
    attention only at the (b, h, t) rows given."""
    st_bf16 = dtype == "bf16"
    f = {n: inp[n].astype(np.float64) for n in "qkvg"}
    if rows is None:
        return oracle.prefill(f["q"], f["k"], f["v"], f["g"], D, W, scale, st_bf16)
    res = {}
    for (b, h) in bh:
        sl = (slice(b, b + 1), slice(h, h + 1))
        hk, sk = oracle.scan(f["g"][sl], f["k"][sl])
        hv, sv = oracle.scan(f["g"][sl], f["v"][sl])
        if st_bf16:
            hk, hv = oracle.round_bf16(hk), oracle.round_bf16(hv)
        ts = [t for (bb, hh, t) in rows if bb == b and hh == h]
        rr = np.array([[0, 0, t] for t in ts], dtype=np.int64)
        o, lse = oracle.attention_rows(f["q"][sl], hk, hv, [D[h]], [W[h]], scale, rr)
        res[(b, h)] = dict(hk=hk[0, 0], hv=hv[0, 0], state_k=sk[0, 0], state_v=sv[0, 0],
                           t=np.array(ts), o=o, lse=lse)
    return res


def sample_rows(T, n=48, seed=0, extra=()):
    rng = np.random.default_rng(seed)
    base = {0, 1, T - 1, T // 2}
    for b in (63, 64, 127, 128, 129, 255, 256):
        if b < T:
            base.add(b)
    base.update(int(x) for x in extra if 0 <= x < T)
    base.update(int(x) for x in rng.integers(0, T, size=n))
    return sorted(base)


def check_cache_layout(out, D, W, T, T_cap, hk_np, hv_np):
    """Kc/Vc and ring hold exactly the GPU's own states at their positions
    (bit-exact), and rows the prefill does not name are untouched (NaN)."""
    R, off = oracle.anchor_offsets(len(D), T_cap, D)
    Kc = out["cache"]["Kc"].float().cpu().numpy()
    Vc = out["cache"]["Vc"].float().cpu().numpy()
    B, H = hk_np.shape[:2]
    for b in range(B):
        for h in range(H):
            n = T // D[h]
            pos = np.arange(n) * D[h] + D[h] - 1
            a0 = off[h]
            np.testing.assert_array_equal(Kc[b, a0:a0 + n], hk_np[b, h, pos])
            np.testing.assert_array_equal(Vc[b, a0:a0 + n], hv_np[b, h, pos])
            assert np.all(np.isnan(Kc[b, a0 + n:off[h + 1]]))
    if sum(W) > 0:
        kr = out["cache"]["k_ring"].float().cpu().numpy()
        vr = out["cache"]["v_ring"].float().cpu().numpy()
        ro = np.concatenate([[0], np.cumsum(W)])
        for b in range(B):
            for h in range(H):
                if W[h] == 0:
                    continue
                written = set()
                for p in range(max(0, T - W[h]), T):
                    s = ro[h] + p % W[h]
                    written.add(s)
                    np.testing.assert_array_equal(kr[b, s], hk_np[b, h, p])
                    np.testing.assert_array_equal(vr[b, s], hv_np[b, h, p])
                for s in range(ro[h], ro[h + 1]):
                    if s not in written:
                        assert np.all(np.isnan(kr[b, s]))


def scale_of(hd):
    return 1.0 / math.sqrt(hd)
