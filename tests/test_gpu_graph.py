"""A step of the hot path (scan, attention, decode) captured into a HIP graph
and replayed gives, on every replay, exactly the results of the same step run
eagerly.  The kernels are deterministic and the scan's workspace tags advance
on the device, so replays need no host-side reset; the library records no
memset or allocation into the graph."""
import numpy as np
import pytest

from dilated_sparse_attention_rat_amd import synth

from gpu_common import say, to_dev

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CASES = [
    # label, B, H, T, hd, D, W  (the first uses the resident-anchor kernel)
    ("resident", 2, 4, 1024, 128, [16, 8, 16, 32], [0, 0, 0, 0]),
    ("window-hybrid", 2, 3, 700, 128, [4, 1, 64], [0, 33, 128]),
]


def _setup(case, seed):
    import dilated_sparse_attention_rat_amd as rat
    label, B, H, T, hd, D, W = case
    inp = synth.random_case(seed, B, H, T + 1, hd, "bf16", hd ** -0.5, 3.0)
    q, k, v, g = (to_dev(np.ascontiguousarray(inp[n][:, :, :T]), "bf16") for n in "qkvg")
    dec = {n: to_dev(np.ascontiguousarray(inp[n][:, :, T]), "bf16") for n in "qkvg"}
    T_cap = T + 1
    c = rat.alloc_cache(B, H, hd, T_cap, D, W, torch.bfloat16, "cuda", fill=0.0)
    s = dict(q=q, k=k, v=v, g=g, dec=dec, c=c, D=D, W=W, T=T, T_cap=T_cap,
             hk=torch.zeros_like(k), hv=torch.zeros_like(v), o=torch.zeros_like(q),
             lse=torch.zeros((B, H, T), dtype=torch.float32, device="cuda"),
             do=torch.zeros_like(dec["q"]), ws=rat.scan_workspace(B, H, T, hd, "cuda"),
             dws=rat.decode_workspace(B, H, hd, T_cap, D, W, "cuda"))
    return s


def _step(s):
    import dilated_sparse_attention_rat_amd as rat
    c, D, W, T, T_cap = s["c"], s["D"], s["W"], s["T"], s["T_cap"]
    rat.rat_scan_prefill(s["k"], s["v"], s["g"], D, W, T_cap, c["Kc"], c["Vc"], c["state_k"],
                         c["state_v"], s["ws"], hk=s["hk"], hv=s["hv"], k_ring=c["k_ring"],
                         v_ring=c["v_ring"])
    rat.rat_dilated_attn_prefill(s["q"], s["hk"], s["hv"], c["Kc"], c["Vc"], D, W, T_cap, s["o"],
                                 s["lse"])
    d = s["dec"]
    rat.rat_decode_step(d["q"], d["k"], d["v"], d["g"], c["state_k"], c["state_v"], c["Kc"],
                        c["Vc"], c["k_ring"], c["v_ring"], s["do"], D, W, T, T_cap,
                        workspace=s["dws"])


def _snapshot(s):
    out = {n: s[n].clone() for n in ("hk", "hv", "o", "lse", "do")}
    out.update({n: t.clone() for n, t in s["c"].items() if t is not None})
    return out


def _clear(s):
    for n in ("hk", "hv", "o", "lse", "do"):
        s[n].zero_()
    for t in s["c"].values():
        if t is not None:
            t.zero_()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager_step(case):
    say(f"[graph] {case[0]}")
    s = _setup(case, 11)
    other = _setup(case, 12)        # eager work on other buffers between replays
    _step(s)
    torch.cuda.synchronize()
    ref = _snapshot(s)
    assert int(s["ws"][2].item()) == 0

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(s)
    torch.cuda.synchronize()
    for rep in range(4):
        _clear(s)
        _step(other)                 # eager launches and a sync between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(s)
        for n, t in ref.items():
            assert torch.equal(got[n], t), f"replay {rep}: {n} differs from the eager step"
        assert int(s["ws"][2].item()) == 0, "scan workspace reports a timed-out wait"
        say(f"  replay {rep}: identical")


def test_graph_topk_decode_replays_equal_eager():
    """Scan, history build and a top-k block decode step, captured and
    replayed, equal the eager step bit for bit (history, block means, the
    selection, o and the caches)."""
    import dilated_sparse_attention_rat_amd as rat
    case = ("topk", 2, 3, 700, 128, [4, 1, 64], [0, 33, 128])
    say("[graph] topk decode")

    def setup(seed):
        s = _setup(case, seed)
        B, H, hd = s["dec"]["q"].shape
        s["hist"] = rat.alloc_topk_history(B, H, hd, s["T_cap"], torch.bfloat16, "cuda", fill=0.0)
        s["sel"] = torch.zeros((B, H, 4), dtype=torch.int32, device="cuda")
        return s

    def step(s):
        c, D, W, T, T_cap, h = s["c"], s["D"], s["W"], s["T"], s["T_cap"], s["hist"]
        rat.rat_scan_prefill(s["k"], s["v"], s["g"], D, W, T_cap, c["Kc"], c["Vc"], c["state_k"],
                             c["state_v"], s["ws"], hk=s["hk"], hv=s["hv"], k_ring=c["k_ring"],
                             v_ring=c["v_ring"])
        rat.rat_topk_cache_build(s["hk"], s["hv"], h["hk_hist"], h["hv_hist"], h["block_means"])
        d = s["dec"]
        rat.rat_decode_step_topk(d["q"], d["k"], d["v"], d["g"], c["state_k"], c["state_v"],
                                 c["Kc"], c["Vc"], c["k_ring"], c["v_ring"], h["hk_hist"],
                                 h["hv_hist"], h["block_means"], s["do"], D, W, T, T_cap, 4,
                                 sel_out=s["sel"])

    def snap(s):
        out = {n: s[n].clone() for n in ("hk", "hv", "do", "sel")}
        out.update({n: t.clone() for n, t in s["c"].items() if t is not None})
        out.update({n: t.clone() for n, t in s["hist"].items()})
        return out

    def clear(s):
        _clear(s)
        s["sel"].zero_()
        for t in s["hist"].values():
            t.zero_()

    s, other = setup(13), setup(14)
    step(s)
    torch.cuda.synchronize()
    ref = snap(s)
    assert int((ref["sel"] >= 0).sum().item()) > 0, "no block was selected"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(s)
    torch.cuda.synchronize()
    for rep in range(4):
        clear(s)
        step(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snap(s)
        for n, t in ref.items():
            assert torch.equal(got[n], t), f"replay {rep}: {n} differs from the eager step"
        assert int(s["ws"][2].item()) == 0, "scan workspace reports a timed-out wait"
        say(f"  replay {rep}: identical")
