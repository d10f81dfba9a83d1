"""GPU parity of chunked prefill: a sequence processed as consecutive chunks
(rat_scan_prefill_continue + rat_dilated_attn_prefill_continue, the state and
the window ring carried from chunk to chunk) against the oracle's prefill of
the whole sequence, through the C ABI.  Two ring buffers are used alternately:
each chunk's attention reads the window positions before the chunk from the
ring the previous chunk left."""
import zlib

import numpy as np
import pytest

import oracle
from dilated_sparse_attention_rat_amd import synth

from gpu_common import (Checks, check_float, check_fp32_state, check_state_ulp, oracle_prefill,
                        say, scale_of, to_dev, to_np)

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

NAN = float("nan")


def _run_chunks(inp, chunks, D, W, T_cap, dtype, first_plain=True, decode_steps=0):
    """Run the chunks on the GPU; returns per-chunk outputs and the final
    cache (the last chunk's ring is the live one)."""
    import dilated_sparse_attention_rat_amd as rat
    B, H, Ttot, hd = inp["q"].shape
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    R, _ = rat.rat_anchor_rows(H, T_cap, D)
    WS, _ = rat.rat_ring_rows(H, W)
    Kc = torch.full((B, R, hd), NAN, dtype=st, device="cuda")
    Vc = torch.full_like(Kc, NAN)
    rings = [(torch.full((B, WS, hd), NAN, dtype=st, device="cuda"),
              torch.full((B, WS, hd), NAN, dtype=st, device="cuda")) if WS > 0 else (None, None)
             for _ in range(2)]
    states = [(torch.full((B, H, hd), NAN, dtype=torch.float32, device="cuda"),
               torch.full((B, H, hd), NAN, dtype=torch.float32, device="cuda")) for _ in range(2)]
    states[1][0].zero_()
    states[1][1].zero_()   # input state of a first chunk run through the continuation
    hks, hvs, os_, lses = [], [], [], []
    t0 = 0
    cur = 0
    for i, T in enumerate(chunks):
        say(f"  chunk {i}: t0={t0} T={T}")
        sl = slice(t0, t0 + T)
        q, k, v, g = (to_dev(np.ascontiguousarray(inp[n][:, :, sl]), dtype) for n in "qkvg")
        hk = torch.full_like(k, NAN)
        hv = torch.full_like(v, NAN)
        ws = rat.scan_workspace(B, H, T, hd, "cuda")
        kr, vr = rings[cur]
        sk, sv = states[cur]
        pk, pv = rings[1 - cur]
        pk_s, pv_s = states[1 - cur]
        if i == 0 and first_plain:
            rat.rat_scan_prefill(k, v, g, D, W, T_cap, Kc, Vc, sk, sv, ws, hk=hk, hv=hv,
                                 k_ring=kr, v_ring=vr)
        else:
            rat.rat_scan_prefill_continue(k, v, g, D, W, T_cap, t0, pk_s, pv_s, Kc, Vc, sk, sv,
                                          ws, hk=hk, hv=hv, k_ring_in=pk if t0 > 0 else None,
                                          v_ring_in=pv if t0 > 0 else None, k_ring=kr, v_ring=vr)
        o = torch.full_like(q, NAN)
        lse = torch.full((B, H, T), NAN, dtype=torch.float32, device="cuda")
        if i == 0 and first_plain:
            rat.rat_dilated_attn_prefill(q, hk, hv, Kc, Vc, D, W, T_cap, o, lse)
        else:
            rat.rat_dilated_attn_prefill_continue(q, hk, hv, Kc, Vc, D, W, T_cap, t0, o,
                                                  k_ring_prev=pk if t0 > 0 else None,
                                                  v_ring_prev=pv if t0 > 0 else None, lse=lse)
        torch.cuda.synchronize()
        assert int(ws[2].item()) == 0, "scan workspace reports a timed-out wait"
        hks.append(hk)
        hvs.append(hv)
        os_.append(o)
        lses.append(lse)
        # the next chunk writes the other ring / state and reads these
        cur = 1 - cur
        t0 += T
    kr, vr = rings[1 - cur]
    sk, sv = states[1 - cur]
    dec = []
    if decode_steps:
        dws = rat.decode_workspace(B, H, hd, T_cap, D, W, "cuda")
        for s in range(decode_steps):
            pos = t0 + s
            q, k, v, g = (to_dev(inp[n][:, :, pos], dtype) for n in "qkvg")
            o = torch.full_like(q, NAN)
            rat.rat_decode_step(q, k, v, g, sk, sv, Kc, Vc, kr, vr, o, D, W, pos, T_cap,
                                workspace=dws)
            dec.append(o)
        torch.cuda.synchronize()
    return dict(hk=to_np(torch.cat(hks, dim=2)), hv=to_np(torch.cat(hvs, dim=2)),
                o=to_np(torch.cat(os_, dim=2)), lse=to_np(torch.cat(lses, dim=2)),
                Kc=to_np(Kc), Vc=to_np(Vc), kr=None if kr is None else to_np(kr),
                vr=None if vr is None else to_np(vr), sk=to_np(sk), sv=to_np(sv),
                dec=to_np(torch.stack(dec, dim=2)) if dec else None, T=t0)



def _run_chunks_two_streams(inp, chunks, D, W, T_cap, dtype):
    """The chunks of _run_chunks (first chunk through the plain entry points)
    as a two-stream pipeline: chunk i's scan on one stream beside chunk
    i-1's attention on the other.  Three rings and two hk/hv buffers are
    used in turn, so the scan of chunk i waits only for the attention of
    chunk i-2, the last reader of the ring and state buffers it overwrites
    (each attention reads the ring of the chunk before it)."""
    import dilated_sparse_attention_rat_amd as rat
    B, H, Ttot, hd = inp["q"].shape
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    R, _ = rat.rat_anchor_rows(H, T_cap, D)
    WS, _ = rat.rat_ring_rows(H, W)
    Kc = torch.full((B, R, hd), NAN, dtype=st, device="cuda")
    Vc = torch.full_like(Kc, NAN)
    rings = [(torch.full((B, WS, hd), NAN, dtype=st, device="cuda"),
              torch.full((B, WS, hd), NAN, dtype=st, device="cuda")) if WS > 0 else (None, None)
             for _ in range(3)]
    states = [(torch.full((B, H, hd), NAN, dtype=torch.float32, device="cuda"),
               torch.full((B, H, hd), NAN, dtype=torch.float32, device="cuda")) for _ in range(2)]
    n = len(chunks)
    starts = np.concatenate([[0], np.cumsum(chunks)]).astype(int)
    ins = [{k: to_dev(np.ascontiguousarray(inp[k][:, :, starts[i]:starts[i + 1]]), dtype)
            for k in "qkvg"} for i in range(n)]
    tmax = max(chunks)
    hkv = [(torch.empty(B * H * tmax * hd, dtype=st, device="cuda"),
            torch.empty(B * H * tmax * hd, dtype=st, device="cuda")) for _ in range(2)]
    wss = [rat.scan_workspace(B, H, T, hd, "cuda") for T in chunks]
    os_ = [torch.full_like(ins[i]["q"], NAN) for i in range(n)]
    lses = [torch.full((B, H, chunks[i]), NAN, dtype=torch.float32, device="cuda") for i in range(n)]
    torch.cuda.synchronize()
    s_scan, s_attn = torch.cuda.Stream(), torch.cuda.Stream()
    ev_s = [torch.cuda.Event() for _ in range(n)]
    ev_a = [torch.cuda.Event() for _ in range(n)]
    for i in range(n):
        t0, T = int(starts[i]), chunks[i]
        cur, prev = rings[i % 3], rings[(i - 1) % 3]
        sc, sp = states[i % 2], states[1 - i % 2]
        hk, hv = (x[:B * H * T * hd].view(B, H, T, hd) for x in hkv[i % 2])
        say(f"  chunk {i}: t0={t0} T={T} (two streams)")
        with torch.cuda.stream(s_scan):
            if i >= 2:
                s_scan.wait_event(ev_a[i - 2])
            x = ins[i]
            if i == 0:
                rat.rat_scan_prefill(x["k"], x["v"], x["g"], D, W, T_cap, Kc, Vc, sc[0], sc[1],
                                     wss[i], hk=hk, hv=hv, k_ring=cur[0], v_ring=cur[1])
            else:
                rat.rat_scan_prefill_continue(x["k"], x["v"], x["g"], D, W, T_cap, t0, sp[0], sp[1],
                                              Kc, Vc, sc[0], sc[1], wss[i], hk=hk, hv=hv,
                                              k_ring_in=prev[0], v_ring_in=prev[1], k_ring=cur[0],
                                              v_ring=cur[1])
            ev_s[i].record(s_scan)
        with torch.cuda.stream(s_attn):
            s_attn.wait_event(ev_s[i])
            if i == 0:
                rat.rat_dilated_attn_prefill(x["q"], hk, hv, Kc, Vc, D, W, T_cap, os_[i], lses[i])
            else:
                rat.rat_dilated_attn_prefill_continue(x["q"], hk, hv, Kc, Vc, D, W, T_cap, t0, os_[i],
                                                      k_ring_prev=prev[0], v_ring_prev=prev[1],
                                                      lse=lses[i])
            ev_a[i].record(s_attn)
    torch.cuda.synchronize()
    for ws in wss:
        assert int(ws[2].item()) == 0, "scan workspace reports a timed-out wait"
    kr, vr = rings[(n - 1) % 3]
    sk, sv = states[(n - 1) % 2]
    return dict(o=to_np(torch.cat(os_, dim=2)), lse=to_np(torch.cat(lses, dim=2)), Kc=to_np(Kc),
                Vc=to_np(Vc), kr=None if kr is None else to_np(kr),
                vr=None if vr is None else to_np(vr), sk=to_np(sk), sv=to_np(sv))

def _check_layout(chk, out, D, W, T_cap):
    """Anchor rows and the live ring hold the GPU's own states at their
    positions (bit-exact); anchor rows beyond the sequence stay untouched."""
    T = out["T"]
    B, H = out["hk"].shape[:2]
    R, off = oracle.anchor_offsets(H, T_cap, D)
    ro = np.concatenate([[0], np.cumsum(W)])

    def layout():
        for b in range(B):
            for h in range(H):
                n = T // D[h]
                pos = np.arange(n) * D[h] + D[h] - 1
                np.testing.assert_array_equal(out["Kc"][b, off[h]:off[h] + n], out["hk"][b, h, pos])
                np.testing.assert_array_equal(out["Vc"][b, off[h]:off[h] + n], out["hv"][b, h, pos])
                assert np.all(np.isnan(out["Kc"][b, off[h] + n:off[h + 1]]))
                if W[h] == 0:
                    continue
                written = set()
                for p in range(max(0, T - W[h]), T):
                    s = ro[h] + p % W[h]
                    written.add(s)
                    np.testing.assert_array_equal(out["kr"][b, s], out["hk"][b, h, p])
                    np.testing.assert_array_equal(out["vr"][b, s], out["hv"][b, h, p])
                for s in range(ro[h], ro[h + 1]):
                    if s not in written:
                        assert np.all(np.isnan(out["kr"][b, s]))

    chk(layout)


CASES = [
    # label, B, H, chunks, hd, D, W, dtype, T_cap extra, first chunk plain
    ("bf16-hybrid-long-chunks", 2, 3, [300, 200, 77], 128, [4, 1, 16], [0, 37, 3], "bf16", 5, True),
    ("bf16-chunks-shorter-than-window", 1, 2, [100, 5, 3, 1, 40], 128, [3, 8], [64, 0], "bf16", 0,
     True),
    ("f32-64", 1, 2, [130, 70], 64, [2, 7], [5, 100], "f32", 3, False),
    ("bf16-resident-anchors", 1, 2, [700, 1300], 128, [16, 64], [0, 0], "bf16", 0, True),
    ("bf16-empty-middle-chunk", 1, 2, [50, 0, 30], 64, [4, 1], [6, 2], "bf16", 0, False),
    ("bf16-unaligned-boundaries", 2, 2, [129, 255, 63], 128, [5, 2], [0, 130], "bf16", 9, True),
    # continuation chunks whose average key set is 512 or more: the launch with
    # two query blocks per wave reading the previous call's ring
    ("qb2-ring-bf16", 1, 2, [700, 600], 128, [1, 1], [300, 0], "bf16", 0, True),
    ("qb2-ring-f32", 1, 2, [600, 500], 64, [1, 2], [200, 0], "f32", 4, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunked_prefill_equals_whole_sequence(case):
    label, B, H, chunks, hd, D, W, dtype, extra, first_plain = case
    T = sum(chunks)
    say(f"[chunked] {label}: B={B} H={H} chunks={chunks} hd={hd} D={D} W={W} {dtype}")
    std = 1.0 if dtype == "f32" else hd ** -0.5
    inp = synth.random_case(zlib.crc32(label.encode()) % 1000, B, H, T, hd, dtype, std, 3.0)
    D, W = np.array(D, np.int32), np.array(W, np.int32)
    T_cap = T + extra
    out = _run_chunks(inp, chunks, D, W, T_cap, dtype, first_plain)
    ref = oracle_prefill(inp, D, W, scale_of(hd), dtype)
    chk = Checks()
    chk(check_state_ulp, "hk", out["hk"], ref["hk"], dtype)
    chk(check_state_ulp, "hv", out["hv"], ref["hv"], dtype)
    chk(check_fp32_state, "state_k", out["sk"], ref["state_k"])
    chk(check_fp32_state, "state_v", out["sv"], ref["state_v"])
    chk(check_float, "o", out["o"], ref["o"], dtype)
    chk(check_float, "lse", out["lse"], ref["lse"], dtype, extra_rel=1e-3)
    _check_layout(chk, out, list(D), list(W), T_cap)
    chk.done()


def test_chunked_prefill_then_decode():
    """Decode steps continue from the state, anchors and ring that a chunked
    prefill leaves; they equal the oracle's prefill rows at those positions."""
    B, H, hd, chunks, steps = 1, 3, 128, [90, 45], 20
    D, W = np.array([4, 1, 8], np.int32), np.array([0, 11, 50], np.int32)
    T = sum(chunks)
    say(f"[chunked] then decode: chunks={chunks} steps={steps}")
    inp = synth.random_case(4242, B, H, T + steps, hd, "bf16", hd ** -0.5, 3.0)
    out = _run_chunks(inp, chunks, D, W, T + steps, "bf16", decode_steps=steps)
    ref = oracle_prefill(inp, D, W, scale_of(hd), "bf16")
    chk = Checks()
    chk(check_float, "o(prefill)", out["o"], ref["o"][:, :, :T], "bf16")
    chk(check_float, "o(decode)", out["dec"], ref["o"][:, :, T:], "bf16")
    chk(check_fp32_state, "state_k", out["sk"], ref["state_k"])
    chk.done()


def test_workload_sized_second_chunk_sampled():
    """A 1.5B-like head layout (16 heads, hd 128, D 4..64, no window) whose
    sequence arrives as two 2048-position chunks: sampled rows of the second
    chunk against the oracle."""
    B, H, hd = 1, 16, 128
    D = np.array([4, 8, 16, 32, 64, 4, 8, 16, 32, 64, 4, 8, 16, 32, 64, 16], np.int32)
    W = np.zeros(H, np.int32)
    chunks = [2048, 2048]
    T = sum(chunks)
    say(f"[chunked] sampled: H={H} chunks={chunks}")
    inp = synth.random_case(77, B, H, T, hd, "bf16", hd ** -0.5, 3.0)
    out = _run_chunks(inp, chunks, D, W, T, "bf16")
    rng = np.random.default_rng(5)
    ts = sorted({2048, 2049, 2111, 2112, T - 1} | set(int(x) for x in rng.integers(2048, T, 24)))
    bh = [(0, h) for h in (0, 4, 9, 15)]
    rows = [(b, h, t) for (b, h) in bh for t in ts]
    ref = oracle_prefill(inp, D, W, scale_of(hd), "bf16", rows=rows, bh=bh)
    chk = Checks()
    for (b, h) in bh:
        r = ref[(b, h)]
        chk(check_float, f"o[{b},{h}]", out["o"][b, h, r["t"]], r["o"], "bf16")
        chk(check_state_ulp, f"hk[{b},{h}]", out["hk"][b, h, 2048:], r["hk"][2048:], "bf16")
    chk.done()


PIPE = [
    # label, B, H, chunks, hd, D, W
    ("hybrid-window", 2, 3, [300, 200, 77, 150], 128, [4, 1, 16], [0, 37, 3]),
    ("chunks-shorter-than-window", 1, 2, [100, 5, 3, 1, 40, 64], 128, [3, 8], [64, 0]),
]


@pytest.mark.parametrize("case", PIPE, ids=[c[0] for c in PIPE])
def test_two_stream_pipeline_equals_one_stream(case):
    """Chunk i's scan on a second stream beside chunk i-1's attention gives
    the outputs, anchors, final state and live ring of the one-stream chunk
    sequence, bit for bit (the kernels are deterministic and the buffer
    rotation leaves no read of a buffer that a concurrent launch writes)."""
    label, B, H, chunks, hd, D, W = case
    T = sum(chunks)
    say(f"[chunked] two streams {label}: B={B} H={H} chunks={chunks} D={D} W={W}")
    inp = synth.random_case(zlib.crc32(label.encode()) % 1000, B, H, T, hd, "bf16", hd ** -0.5, 3.0)
    D, W = np.array(D, np.int32), np.array(W, np.int32)
    one = _run_chunks(inp, chunks, D, W, T, "bf16", True)
    two = _run_chunks_two_streams(inp, chunks, D, W, T, "bf16")
    for k in ("o", "lse", "Kc", "Vc", "kr", "vr", "sk", "sv"):
        if one[k] is None:
            assert two[k] is None, k
            continue
        np.testing.assert_array_equal(np.nan_to_num(two[k], nan=7.0), np.nan_to_num(one[k], nan=7.0),
                                      err_msg=k)
