"""GPU parity of the top-k block decode step (history cache build, block
scoring and selection, attention over anchors + window + selected blocks, the
step's cache writes) against the oracle.

The selection is an integer decision taken from fp32 scores of block means
that the GPU computes from its own stored (bf16 or fp32) states, while the
oracle scores in fp64 from its own rounded states.  So the GPU's selection is
checked for validity under the oracle's scores -- the right count, distinct,
eligible, and every selected block scoring at least as high as every
unselected one up to the bound on the score's error -- and the output is then
compared with the oracle's step on the GPU's selection.  Score error bound per
block m (q the query, A[m,i] the mean |stored state| of the block in channel
i, S the largest |stored state| of the head): bf16 storage
sum_i |q_i| (2^-7 A[m,i] + 2^-15 S), one storage ulp per row plus the fp32
rounding of the row sum and the dot product; fp32 storage
sum_i |q_i| (1e-5 A[m,i] + 2^-18 S + 1e-6)."""
import numpy as np
import pytest

import oracle
from dilated_sparse_attention_rat_amd import synth

from gpu_common import (Checks, check_float, check_fp32_state, check_state_ulp, gpu_prefill, say,
                        scale_of, to_dev, to_np, torch_dtype)

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

BLK = oracle.TOPK_BLOCK


def _score_tol(q, hist, ne, dtype):
    """Per-block bound on |GPU score - oracle score| (see the module docstring)."""
    if ne == 0:
        return np.zeros(0)
    A = np.abs(hist[:ne * BLK]).reshape(ne, BLK, -1).mean(axis=1)
    S = float(np.abs(hist).max()) if hist.size else 0.0
    aq = np.abs(q)
    if dtype == "bf16":
        return (2.0 ** -7 * A + 2.0 ** -15 * S) @ aq
    return (1e-5 * A + 2.0 ** -18 * S + 1e-6) @ aq


def check_selection(name, sel, k_sel, scores, tol, own):
    """sel: the GPU's [k_sel] entries; scores/tol: oracle scores and bounds of
    the eligible blocks; own: the oracle's own selection.  Returns True when
    the GPU picked the same set as the oracle."""
    ne = len(scores)
    ks = min(k_sel, ne)
    picked = [int(m) for m in sel[:ks]]
    assert all(int(m) == -1 for m in sel[ks:]), f"{name}: entries past {ks} not -1: {sel}"
    assert len(set(picked)) == ks and all(0 <= m < ne for m in picked), \
        f"{name}: not {ks} distinct eligible blocks: {sel} (eligible {ne})"
    rest = np.setdiff1d(np.arange(ne), picked)
    if ks and rest.size:
        lo_sel = float(np.min(scores[picked] + tol[picked]))
        hi_rest = float(np.max(scores[rest] - tol[rest]))
        assert lo_sel >= hi_rest, \
            f"{name}: an unselected block scores above a selected one beyond the bound " \
            f"({lo_sel} < {hi_rest})"
    return set(picked) == set(int(m) for m in own)


def check_means(name, got, hist, n_blocks, dtype):
    """Block means of the GPU's history against the oracle's rounded states."""
    if n_blocks == 0:
        return
    ref = oracle.block_means(hist[None, None, :n_blocks * BLK])[0, 0]
    A = np.abs(hist[:n_blocks * BLK]).reshape(n_blocks, BLK, -1).mean(axis=1)
    S = float(np.abs(hist).max())
    lim = (2.0 ** -7 * A + 2.0 ** -15 * S) if dtype == "bf16" else (1e-5 * A + 2.0 ** -18 * S + 1e-7)
    d = np.abs(np.asarray(got, np.float64) - ref)
    say(f"  {name}: max|err|={d.max():.3e} ({int((d > lim).sum())} beyond the bound)")
    assert np.all(d <= lim), f"{name}: {int((d > lim).sum())} values beyond the bound"


def _gpu_chain(inp, T, steps, D, W, T_cap, k_sel, dtype):
    import dilated_sparse_attention_rat_amd as rat
    B, H, _, hd = inp["q"].shape
    pre = {n: np.ascontiguousarray(inp[n][:, :, :T]) for n in "qkvg"}
    out = gpu_prefill(pre, D, W, T_cap, dtype, with_hk=T > 0)
    c = out["cache"]
    hist = rat.alloc_topk_history(B, H, hd, T_cap, torch_dtype(dtype), "cuda", fill=float("nan"))
    if T > 0:
        rat.rat_topk_cache_build(out["hk_t"], out["hv_t"], hist["hk_hist"], hist["hv_hist"],
                                 hist["block_means"])
    os_, sels = [], []
    for s in range(steps):
        pos = T + s
        q, k, v, g = (to_dev(inp[n][:, :, pos], dtype) for n in "qkvg")
        o = torch.empty_like(q)
        sel = torch.full((B, H, k_sel), -7, dtype=torch.int32, device="cuda") if k_sel else None
        rat.rat_decode_step_topk(q, k, v, g, c["state_k"], c["state_v"], c["Kc"], c["Vc"],
                                 c["k_ring"], c["v_ring"], hist["hk_hist"], hist["hv_hist"],
                                 hist["block_means"], o, D, W, pos, T_cap, k_sel, sel_out=sel)
        os_.append(o)
        sels.append(sel)
    torch.cuda.synchronize()
    o = to_np(torch.stack(os_, dim=2))
    sel = (torch.stack(sels, dim=2).cpu().numpy() if k_sel
           else np.zeros((B, H, steps, 0), np.int64))
    return o, sel, c, hist


CASES = [
    # label, B, H, T, hd, D, W, dtype, steps, T_cap, k
    ("bf16-128-mixed", 2, 3, 300, 128, [4, 1, 16], [0, 40, 7], "bf16", 40, 400, 3),
    ("f32-64", 1, 2, 200, 64, [5, 2], [0, 64], "f32", 60, 300, 2),
    ("k-exceeds-blocks", 1, 2, 130, 128, [8, 3], [0, 0], "bf16", 70, 256, 10),
    ("from-empty", 1, 2, 0, 128, [3, 1], [5, 0], "bf16", 140, 200, 2),
    ("k0-dilated-only", 1, 2, 260, 64, [4, 16], [0, 9], "bf16", 8, 300, 0),
    ("hd64-many-blocks", 2, 2, 1500, 64, [16, 2], [64, 0], "bf16", 6, 1600, 8),
    ("f32-128-dense-wide", 1, 2, 700, 128, [1, 32], [600, 300], "f32", 5, 760, 4),
    ("k-max", 1, 1, 5000, 128, [64], [128], "bf16", 3, 5100, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_topk_decode_steps(case):
    label, B, H, T, hd, D, W, dtype, steps, T_cap, k_sel = case
    say(f"[topk] {label}: B={B} H={H} T={T} steps={steps} D={D} W={W} {dtype} k={k_sel}")
    std = 1.0 if dtype == "f32" else hd ** -0.5
    inp = synth.random_case(len(label) * 11 + T, B, H, T + steps, hd, dtype, std, 3.0)
    D, W = np.array(D, np.int32), np.array(W, np.int32)
    o, sel, c, hist = _gpu_chain(inp, T, steps, D, W, T_cap, k_sel, dtype)
    _check_steps(inp, T, steps, D, W, T_cap, k_sel, dtype, o, sel, c, hist)


def _check_steps(inp, T, steps, D, W, T_cap, k_sel, dtype, o, sel, c, hist):
    """Decode steps at positions T .. T+steps-1 (GPU output o, selections sel,
    final cache c and history hist) against the oracle over the whole input."""
    B, H, _, hd = inp["q"].shape
    n = T + steps
    f = {x: inp[x][:, :, :n].astype(np.float64) for x in "qkvg"}
    hk_u, sk = oracle.scan(f["g"], f["k"])
    hv_u, sv = oracle.scan(f["g"], f["v"])
    hk, hv = (oracle.round_bf16(hk_u), oracle.round_bf16(hv_u)) if dtype == "bf16" else (hk_u, hv_u)
    chk = Checks()
    ref_o = np.empty_like(o)
    same, total = 0, 0
    for s in range(steps):
        pos = T + s
        zero = np.zeros((B, H, hd))
        psk = hk_u[:, :, pos - 1] if pos > 0 else zero
        psv = hv_u[:, :, pos - 1] if pos > 0 else zero
        args = (f["q"][:, :, pos], f["k"][:, :, pos], f["v"][:, :, pos], f["g"][:, :, pos],
                psk, psv, hk[:, :, :pos], hv[:, :, :pos], D, W, scale_of(hd), pos, k_sel,
                dtype == "bf16")
        own = oracle.decode_step_topk(*args)
        for b in range(B):
            for h in range(H):
                ne = int(own["n_elig"][b, h])
                tol = _score_tol(f["q"][b, h, pos], hk[b, h, :pos], ne, dtype)
                same += check_selection(f"sel[{b},{h},pos={pos}]", sel[b, h, s], k_sel,
                                        own["scores"][(b, h)], tol, own["sel"][b, h][own["sel"][b, h] >= 0])
                total += 1
        r = oracle.decode_step_topk(*args, sel=sel[:, :, s] if k_sel else None)
        ref_o[:, :, s] = r["o"]
    say(f"  selection equal to the oracle's own in {same} of {total} (b, h, step)")
    chk(check_float, "o", o, ref_o, dtype)
    chk(check_fp32_state, "state_k", to_np(c["state_k"]), sk)
    chk(check_fp32_state, "state_v", to_np(c["state_v"]), sv)
    ghk, ghv = to_np(hist["hk_hist"]), to_np(hist["hv_hist"])
    chk(check_state_ulp, "hk_hist", ghk[:, :, :n], hk, dtype)
    chk(check_state_ulp, "hv_hist", ghv[:, :, :n], hv, dtype)
    assert np.all(np.isnan(ghk[:, :, n:])), "history rows past the last step were written"
    gm = to_np(hist["block_means"])
    nb = n // BLK
    for b in range(B):
        for h in range(H):
            chk(check_means, f"means[{b},{h}]", gm[b, h, :nb], hk[b, h], nb, dtype)
    assert np.all(np.isnan(gm[:, :, nb:])), "means of incomplete blocks were written"
    R, off = oracle.anchor_offsets(H, T_cap, D)
    Kc = to_np(c["Kc"])
    for b in range(B):
        for h in range(H):
            na = n // D[h]
            p = np.arange(na) * D[h] + D[h] - 1
            chk(check_state_ulp, f"Kc[{b},{h}]", Kc[b, off[h]:off[h] + na], hk[b, h, p], dtype)
    chk.done()


CHUNK_CASES = [
    # label, B, H, chunks, hd, D, W, dtype, steps, T_cap, k
    ("chunks-bf16", 1, 2, [150, 170, 40], 128, [4, 2], [0, 30], "bf16", 30, 420, 3),
    ("chunks-f32-64", 2, 2, [64, 100], 64, [8, 1], [16, 0], "f32", 20, 200, 2),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_topk_decode_after_chunked_prefill(case):
    """A chunked prefill (continuation entry points) whose history is built
    chunk by chunk (the chunk start t0 given; blocks that straddle a chunk
    boundary get their mean when the later chunk completes them), then top-k
    decode steps, against the oracle over the whole sequence."""
    import dilated_sparse_attention_rat_amd as rat
    label, B, H, chunks, hd, D, W, dtype, steps, T_cap, k_sel = case
    T = sum(chunks)
    say(f"[topk] {label}: B={B} H={H} chunks={chunks} steps={steps} D={D} W={W} {dtype}")
    std = 1.0 if dtype == "f32" else hd ** -0.5
    inp = synth.random_case(len(label) * 13 + T, B, H, T + steps, hd, dtype, std, 3.0)
    D, W = np.array(D, np.int32), np.array(W, np.int32)
    st = torch_dtype(dtype)
    c = rat.alloc_cache(B, H, hd, T_cap, D, W, st, "cuda", fill=float("nan"))
    hist = rat.alloc_topk_history(B, H, hd, T_cap, st, "cuda", fill=float("nan"))
    rings = [(c["k_ring"], c["v_ring"]),
             (torch.full_like(c["k_ring"], float("nan")) if c["k_ring"] is not None else None,
              torch.full_like(c["v_ring"], float("nan")) if c["v_ring"] is not None else None)]
    states = [(c["state_k"], c["state_v"]),
              (torch.zeros_like(c["state_k"]), torch.zeros_like(c["state_v"]))]
    t0, cur = 0, 0
    for T_i in chunks:
        k, v, g = (to_dev(np.ascontiguousarray(inp[x][:, :, t0:t0 + T_i]), dtype) for x in "kvg")
        hk, hv = torch.empty_like(k), torch.empty_like(v)
        ws = rat.scan_workspace(B, H, T_i, hd, "cuda")
        (kr, vr), (pk, pv) = rings[cur], rings[1 - cur]
        (sk, sv), (psk, psv) = states[cur], states[1 - cur]
        rat.rat_scan_prefill_continue(k, v, g, D, W, T_cap, t0, psk, psv, c["Kc"], c["Vc"], sk,
                                      sv, ws, hk=hk, hv=hv,
                                      k_ring_in=pk if t0 > 0 else None,
                                      v_ring_in=pv if t0 > 0 else None, k_ring=kr, v_ring=vr)
        rat.rat_topk_cache_build(hk, hv, hist["hk_hist"], hist["hv_hist"], hist["block_means"],
                                 t0=t0)
        torch.cuda.synchronize()
        assert int(ws[2].item()) == 0
        t0 += T_i
        cur = 1 - cur
    (kr, vr), (sk, sv) = rings[1 - cur], states[1 - cur]
    os_, sels = [], []
    for s in range(steps):
        pos = T + s
        q, k, v, g = (to_dev(inp[x][:, :, pos], dtype) for x in "qkvg")
        o = torch.empty_like(q)
        sel = torch.full((B, H, k_sel), -7, dtype=torch.int32, device="cuda")
        rat.rat_decode_step_topk(q, k, v, g, sk, sv, c["Kc"], c["Vc"], kr, vr, hist["hk_hist"],
                                 hist["hv_hist"], hist["block_means"], o, D, W, pos, T_cap,
                                 k_sel, sel_out=sel)
        os_.append(o)
        sels.append(sel)
    torch.cuda.synchronize()
    o = to_np(torch.stack(os_, dim=2))
    sel = torch.stack(sels, dim=2).cpu().numpy()
    _check_steps(inp, T, steps, D, W, T_cap, k_sel, dtype, o, sel,
                 dict(state_k=sk, state_v=sv, Kc=c["Kc"]), hist)


def test_topk_matches_plain_decode_when_nothing_is_selected():
    """k = 0 through the top-k entry point equals the plain decode step's output."""
    import dilated_sparse_attention_rat_amd as rat
    B, H, T, hd, T_cap = 2, 2, 333, 128, 400
    D, W = np.array([4, 7], np.int32), np.array([0, 21], np.int32)
    inp = synth.random_case(77, B, H, T + 4, hd, "bf16", hd ** -0.5, 3.0)
    o_topk = _gpu_chain(inp, T, 4, D, W, T_cap, 0, "bf16")[0]
    pre = {n: np.ascontiguousarray(inp[n][:, :, :T]) for n in "qkvg"}
    c = gpu_prefill(pre, D, W, T_cap, "bf16", with_hk=False)["cache"]
    dws = rat.decode_workspace(B, H, hd, T_cap, D, W, "cuda")
    outs = []
    for s in range(4):
        q, k, v, g = (to_dev(inp[n][:, :, T + s], "bf16") for n in "qkvg")
        o = torch.empty_like(q)
        rat.rat_decode_step(q, k, v, g, c["state_k"], c["state_v"], c["Kc"], c["Vc"],
                            c["k_ring"], c["v_ring"], o, D, W, T + s, T_cap, workspace=dws)
        outs.append(o)
    o_plain = to_np(torch.stack(outs, dim=2))
    d = np.abs(o_topk - o_plain)
    say(f"  topk(k=0) vs plain decode: max|diff|={d.max():.3e}")
    assert d.max() <= 2.0 ** -7 * np.abs(o_plain).max()


def test_topk_decode_workload_full_size_sampled():
    """The decode workload's shape (batch 64, 32 heads, context 32768, D = 64,
    W = 128, 256 steps) with k = 8 blocks, in the benchmark's launch
    configuration; sampled (b, h) are checked step by step against the
    oracle, including the steps that select a block whose mean the decode
    itself wrote."""
    import dilated_sparse_attention_rat_amd as rat
    w = synth.WORKLOADS[3]
    K_SEL = 8
    B, H, T, hd, steps = w.B, w.H, w.T, w.hd, w.decode_steps
    T_cap = w.T_cap
    D, W = np.array(w.D, np.int32), np.array(w.W, np.int32)
    st = torch.bfloat16
    say(f"[topk] decode workload: B={B} H={H} T={T} steps={steps} k={K_SEL}")
    cache = rat.alloc_cache(B, H, hd, T_cap, D, W, st, "cuda", fill=float("nan"))
    hist = rat.alloc_topk_history(B, H, hd, T_cap, st, "cuda")
    ws = rat.scan_workspace(1, H, T, hd, "cuda")
    hk_t = torch.empty((1, H, T, hd), dtype=st, device="cuda")
    hv_t = torch.empty_like(hk_t)
    picks = [(0, 0), (63, 31), (17, 5)]
    ctx = {}
    for b in range(B):
        kvg = synth.decode_context_row(w, b)
        rat.rat_scan_prefill(kvg["k"], kvg["v"], kvg["g"], D, W, T_cap, cache["Kc"][b:b + 1],
                             cache["Vc"][b:b + 1], cache["state_k"][b:b + 1],
                             cache["state_v"][b:b + 1], ws, hk=hk_t, hv=hv_t,
                             k_ring=cache["k_ring"][b:b + 1], v_ring=cache["v_ring"][b:b + 1])
        rat.rat_topk_cache_build(hk_t, hv_t, hist["hk_hist"][b:b + 1], hist["hv_hist"][b:b + 1],
                                 hist["block_means"][b:b + 1])
        for (bb, h) in picks:
            if bb == b:
                ctx[(b, h)] = {n: to_np(kvg[n][0, h]) for n in "kvg"}
        del kvg
    torch.cuda.synchronize()
    assert int(ws[2].item()) == 0
    say("  context built")
    step_in = {key: {n: [] for n in "qkvg"} for key in picks}
    outs = {key: [] for key in picks}
    sels = {key: [] for key in picks}
    sel = torch.empty((B, H, K_SEL), dtype=torch.int32, device="cuda")
    for s in range(steps):
        x = synth.decode_step_inputs(w, s)
        o = torch.empty_like(x["q"])
        rat.rat_decode_step_topk(x["q"], x["k"], x["v"], x["g"], cache["state_k"],
                                 cache["state_v"], cache["Kc"], cache["Vc"], cache["k_ring"],
                                 cache["v_ring"], hist["hk_hist"], hist["hv_hist"],
                                 hist["block_means"], o, D, W, T + s, T_cap, K_SEL, sel_out=sel)
        for (b, h) in picks:
            for n in "qkvg":
                step_in[(b, h)][n].append(x[n][b, h])
            outs[(b, h)].append(o[b, h])
            sels[(b, h)].append(sel[b, h].clone())
    torch.cuda.synchronize()
    say(f"  {steps} steps done")
    chk = Checks()
    for (b, h) in picks:
        si = {n: to_np(torch.stack(step_in[(b, h)][n])) for n in "qkvg"}
        kk = np.concatenate([ctx[(b, h)]["k"], si["k"]])[None, None]
        vv = np.concatenate([ctx[(b, h)]["v"], si["v"]])[None, None]
        gg = np.concatenate([ctx[(b, h)]["g"], si["g"]])[None, None]
        hk_u, sk = oracle.scan(gg, kk)
        hv_u, sv = oracle.scan(gg, vv)
        hk, hv = oracle.round_bf16(hk_u), oracle.round_bf16(hv_u)
        gsel = torch.stack(sels[(b, h)]).cpu().numpy()
        ref_o = np.empty((steps, hd))
        same = 0
        for s in range(steps):
            pos = T + s
            args = (si["q"][s][None, None], si["k"][s][None, None], si["v"][s][None, None],
                    si["g"][s][None, None], hk_u[:, :, pos - 1], hv_u[:, :, pos - 1],
                    hk[:, :, :pos], hv[:, :, :pos], D[h:h + 1], W[h:h + 1], w.scale, pos, K_SEL,
                    True)
            own = oracle.decode_step_topk(*args)
            ne = int(own["n_elig"][0, 0])
            tol = _score_tol(si["q"][s], hk[0, 0, :pos], ne, "bf16")
            same += check_selection(f"sel[{b},{h},pos={pos}]", gsel[s], K_SEL, own["scores"][(0, 0)],
                                    tol, own["sel"][0, 0])
            ref_o[s] = oracle.decode_step_topk(*args, sel=gsel[s][None, None])["o"][0, 0]
        say(f" (b={b}, h={h}) selection equal to the oracle's own in {same} of {steps} steps")
        chk(check_float, "o", to_np(torch.stack(outs[(b, h)])), ref_o, "bf16")
        chk(check_fp32_state, "state_k", to_np(cache["state_k"][b, h]), sk[0, 0])
        gm = to_np(hist["block_means"][b, h])
        nb = (T + steps) // BLK
        chk(check_means, "means", gm[:nb], hk[0, 0], nb, "bf16")
        rows = np.array([0, 63, T - 1, T, T + steps - 1])
        chk(check_state_ulp, "hk_hist", to_np(hist["hk_hist"][b, h])[rows], hk[0, 0, rows], "bf16")
    chk.done()
