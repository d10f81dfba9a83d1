"""GPU parity of the prefill path (scan + fused compaction + dilated
attention) against the CPU oracle, through the C ABI."""
import zlib

import numpy as np
import pytest

import oracle
from dilated_sparse_attention_rat_amd import synth

from gpu_common import (Checks, check_cache_layout, check_float, check_fp32_state, check_state_ulp,
                        gpu_prefill, oracle_prefill, sample_rows, say, scale_of, to_np)

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _full_compare(inp, D, W, T_cap, dtype, label, check_layout=True):
    B, H, T, hd = inp["q"].shape
    say(f"[prefill] {label}: B={B} H={H} T={T} hd={hd} D={list(D)} W={list(W)} {dtype}")
    out = gpu_prefill(inp, D, W, T_cap, dtype)
    ref = oracle_prefill(inp, D, W, scale_of(hd), dtype)
    chk = Checks()
    hk, hv = to_np(out["hk_t"]), to_np(out["hv_t"])
    chk(check_state_ulp, "hk", hk, ref["hk"], dtype)
    chk(check_state_ulp, "hv", hv, ref["hv"], dtype)
    chk(check_fp32_state, "state_k", to_np(out["cache"]["state_k"]), ref["state_k"])
    chk(check_fp32_state, "state_v", to_np(out["cache"]["state_v"]), ref["state_v"])
    chk(check_float, "o", to_np(out["o_t"]), ref["o"], dtype)
    chk(check_float, "lse", to_np(out["lse_t"]), ref["lse"], dtype, extra_rel=1e-3)
    if check_layout:
        chk(check_cache_layout, out, list(D), list(W), T, T_cap, hk, hv)
    chk.done()
    return out


SMALL = [
    # label, B, H, T, hd, D, W, dtype, qkv_std, g_bias, T_cap_extra
    ("ragged-bf16-128", 2, 3, 1000, 128, [5, 1, 16], [0, 37, 3], "bf16", 128 ** -0.5, 3.0, 7),
    ("bf16-64", 1, 2, 777, 64, [3, 64], [0, 200], "bf16", 64 ** -0.5, 3.0, 0),
    ("f32-128", 1, 2, 300, 128, [2, 7], [5, 0], "f32", 1.0, 2.0, 0),
    ("f32-64-window", 2, 2, 260, 64, [4, 9], [300, 1], "f32", 1.0, 2.0, 40),
    ("stress-N01-bf16", 1, 2, 513, 128, [4, 1], [0, 0], "bf16", 1.0, 0.0, 0),
    ("T1", 1, 2, 1, 128, [4, 1], [0, 3], "bf16", 128 ** -0.5, 3.0, 5),
    ("T2-D-beyond-T", 1, 2, 2, 64, [7, 2], [0, 0], "f32", 1.0, 2.0, 0),
    ("T129", 1, 1, 129, 128, [1], [0], "bf16", 128 ** -0.5, 3.0, 0),
    ("T127-window", 1, 1, 127, 128, [3], [64], "bf16", 128 ** -0.5, 3.0, 0),
    # average key set of 512 or more: the MFMA-bound launch (two 16-query
    # blocks per wave), with ragged query tiles, band tiles and both dtypes
    ("qb2-dense-hybrid", 1, 2, 1500, 128, [1, 2], [0, 100], "bf16", 128 ** -0.5, 3.0, 3),
    ("qb2-hd64", 1, 1, 1100, 64, [1], [0], "bf16", 64 ** -0.5, 3.0, 0),
    ("qb2-window-band", 1, 2, 1300, 128, [1, 1], [300, 0], "bf16", 128 ** -0.5, 3.0, 0),
    ("qb2-f32", 1, 1, 1030, 64, [1], [0], "f32", 1.0, 2.0, 0),
    # windowless bf16 hd 128 heads past the resident kernel's 256 anchors:
    # the two-block launch whose K/V tiles go straight into LDS (ragged last
    # query and key tiles, two batch rows)
    ("qb2-dma-windowless", 2, 2, 1500, 128, [1, 3], [0, 0], "bf16", 128 ** -0.5, 3.0, 4),
    # windowless bf16 heads with at most 256 anchors: the resident-anchor
    # kernel at hd = 64 (V staged row-major, transposing fragment reads)
    ("resident-bf16-64", 1, 2, 517, 64, [3, 5], [0, 0], "bf16", 64 ** -0.5, 3.0, 0),
    # a chunk tree of four levels (516 chunks of 64 rows)
    ("scan-tree-4-levels", 1, 1, 33000, 128, [256], [0], "bf16", 128 ** -0.5, 3.0, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_prefill_small_full_oracle(case):
    label, B, H, T, hd, D, W, dtype, std, gb, extra = case
    inp = synth.random_case(zlib.crc32(label.encode()) % 1000, B, H, T, hd, dtype, std, gb)
    _full_compare(inp, np.array(D, np.int32), np.array(W, np.int32), T + extra, dtype, label)


def test_tiny_fp32_workload():
    w = synth.WORKLOADS[0]
    inp = synth.prefill_inputs(w)
    _full_compare(inp, np.array(w.D), np.array(w.W), w.T, w.dtype, w.name)


def test_empty_sequence():
    import dilated_sparse_attention_rat_amd as rat
    say("[prefill] T=0")
    B, H, hd = 2, 3, 128
    D, W = [4, 1, 2], [0, 3, 0]
    cache = rat.alloc_cache(B, H, hd, 16, D, W, torch.bfloat16, "cuda", fill=float("nan"))
    cache["state_k"].fill_(5.0)
    cache["state_v"].fill_(5.0)
    e = torch.empty((B, H, 0, hd), dtype=torch.bfloat16, device="cuda")
    ws = rat.scan_workspace(B, H, 0, hd, "cuda")
    rat.rat_scan_prefill(e, e, e, D, W, 16, cache["Kc"], cache["Vc"], cache["state_k"],
                         cache["state_v"], ws, k_ring=cache["k_ring"], v_ring=cache["v_ring"])
    o = torch.empty_like(e)
    rat.rat_dilated_attn_prefill(e, e, e, cache["Kc"], cache["Vc"], D, W, 16, o)
    torch.cuda.synchronize()
    assert torch.all(cache["state_k"] == 0) and torch.all(cache["state_v"] == 0)
    assert torch.all(torch.isnan(cache["Kc"].float()))


FULL = [1, 2, 4]


@pytest.mark.parametrize("wid", FULL)
def test_workload_full_size_sampled(wid):
    """Full-size workload in the benchmark's launch configuration; the oracle
    checks whole (b, h) states and sampled attention rows."""
    w = synth.WORKLOADS[wid]
    inp = synth.prefill_inputs(w)
    D, W = np.array(w.D, np.int32), np.array(w.W, np.int32)
    say(f"[prefill] workload {wid} {w.name}: B={w.B} H={w.H} T={w.T}")
    out = gpu_prefill(inp, D, W, w.T, w.dtype)
    bh = sorted({(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 2), (0, 1), (w.B - 1, 2)})
    rows = [(b, h, t) for (b, h) in bh for t in sample_rows(w.T, seed=wid * 100 + h + 7 * b)]
    ref = oracle_prefill(inp, D, W, w.scale, w.dtype, rows=rows, bh=bh)
    hk, hv = out["hk_t"], out["hv_t"]
    R, off = oracle.anchor_offsets(w.H, w.T, D)
    chk = Checks()
    for (b, h), r in ref.items():
        say(f" (b={b}, h={h}) D={D[h]} W={W[h]}")
        hk_bh, hv_bh = to_np(hk[b, h]), to_np(hv[b, h])
        chk(check_state_ulp, "hk", hk_bh, r["hk"], w.dtype)
        chk(check_state_ulp, "hv", hv_bh, r["hv"], w.dtype)
        chk(check_fp32_state, "state_k", to_np(out["cache"]["state_k"][b, h]), r["state_k"])
        o = to_np(out["o_t"][b, h])[r["t"]]
        chk(check_float, "o", o, r["o"], w.dtype)
        chk(check_float, "lse", to_np(out["lse_t"][b, h])[r["t"]], r["lse"], w.dtype, extra_rel=1e-3)
        n = w.T // D[h]
        Kc = to_np(out["cache"]["Kc"][b, off[h]:off[h] + n])
        np.testing.assert_array_equal(Kc, hk_bh[np.arange(n) * D[h] + D[h] - 1])
    chk.done()


def test_deterministic_and_workspace_reuse():
    """Two runs on the same workspace are bitwise identical (the scan's carry
    composition order is fixed), and the workspace stays valid across calls
    of different sizes."""
    w = synth.WORKLOADS[1]
    inp = synth.prefill_inputs(w, B=2)
    D, W = np.array(w.D, np.int32), np.array(w.W, np.int32)
    say("[prefill] determinism, workload 1 at B=2")
    import dilated_sparse_attention_rat_amd as rat
    ws = rat.scan_workspace(w.B, w.H, w.T, w.hd, "cuda")
    a = gpu_prefill(inp, D, W, w.T, w.dtype, ws=ws)
    small = synth.random_case(5, 1, 3, 333, 128, "bf16", 128 ** -0.5, 3.0)
    gpu_prefill(small, np.array([2, 3, 4], np.int32), np.array([0, 0, 9], np.int32), 333, "bf16",
                ws=ws)
    b = gpu_prefill(inp, D, W, w.T, w.dtype, ws=ws)
    for key in ("hk_t", "hv_t", "o_t", "lse_t"):
        assert torch.equal(a[key], b[key]), key
    for key in ("Kc", "Vc", "state_k", "state_v"):
        assert torch.equal(a["cache"][key], b["cache"][key]), key


def test_cache_only_mode_matches():
    """hk/hv = NULL writes the same caches and state."""
    inp = synth.random_case(21, 2, 2, 700, 128, "bf16", 128 ** -0.5, 3.0)
    D, W = np.array([8, 3], np.int32), np.array([16, 0], np.int32)
    say("[prefill] cache-only mode")
    a = gpu_prefill(inp, D, W, 800, "bf16")
    b = gpu_prefill(inp, D, W, 800, "bf16", with_hk=False)
    for key in ("Kc", "Vc", "k_ring", "v_ring", "state_k", "state_v"):
        x, y = a["cache"][key], b["cache"][key]
        assert torch.equal(torch.nan_to_num(x.float(), nan=7.0), torch.nan_to_num(y.float(), nan=7.0)), key


def test_position_coded_layout_bit_exact():
    """g = 0 makes every state equal to its input; channels 0-3 carry
    (t mod 256, t div 256, h, b), exact in bf16, so every anchor row and
    ring slot must decode to its own (b, h, position)."""
    B, H, T, hd = 2, 3, 1100, 128
    D, W = [1, 4, 64], [0, 10, 300]
    T_cap = 1200
    t = np.arange(T)
    k = np.zeros((B, H, T, hd), np.float32)
    for b in range(B):
        for h in range(H):
            k[b, h, :, 0] = t % 256
            k[b, h, :, 1] = t // 256
            k[b, h, :, 2] = h
            k[b, h, :, 3] = b
    inp = dict(q=np.zeros_like(k), k=k, v=-k, g=np.zeros_like(k))
    say("[prefill] position-coded layout")
    out = gpu_prefill(inp, np.array(D, np.int32), np.array(W, np.int32), T_cap, "bf16")
    Kc = out["cache"]["Kc"].float().cpu().numpy()
    Vc = out["cache"]["Vc"].float().cpu().numpy()
    R, off = oracle.anchor_offsets(H, T_cap, D)
    for b in range(B):
        for h in range(H):
            for a in range(off[h + 1] - off[h]):
                row = Kc[b, off[h] + a]
                p = a * D[h] + D[h] - 1
                if p < T:
                    assert (row[0], row[1], row[2], row[3]) == (p % 256, p // 256, h, b)
                    assert np.array_equal(Vc[b, off[h] + a], -row)
                else:
                    assert np.all(np.isnan(row))
    kr = out["cache"]["k_ring"].float().cpu().numpy()
    ro = np.concatenate([[0], np.cumsum(W)])
    for b in range(B):
        for h in range(H):
            for p in range(max(0, T - W[h]), T):
                row = kr[b, ro[h] + p % W[h]]
                assert (row[0], row[1], row[2], row[3]) == (p % 256, p // 256, h, b)
