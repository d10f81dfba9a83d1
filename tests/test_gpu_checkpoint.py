"""Checkpoint and resume of the decode state.

The whole decode state of a layer is the fp32 recurrent state (state_k,
state_v), the anchor cache (Kc, Vc), the window ring (k_ring, v_ring) and
the position.  After 100 decode steps the state is copied to host memory,
restored into freshly allocated buffers, and decoding continues for 28
steps; outputs and the final state must equal, bit for bit, those of the run
that was never interrupted (the kernels are deterministic and read nothing
else).  The uninterrupted run is also compared with the oracle's prefill
rows, so the resumed one is correct too."""
import numpy as np
import pytest

import oracle
from dilated_sparse_attention_rat_amd import synth

from gpu_common import Checks, check_float, gpu_prefill, say, scale_of, to_dev, to_np

torch = pytest.importorskip("torch")
pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

STATE = ("state_k", "state_v", "Kc", "Vc", "k_ring", "v_ring")


@pytest.mark.parametrize("splits", [0, 3], ids=["auto-splits", "splits-3"])
def test_decode_resume_from_host_copy_is_bitwise_identical(splits):
    import dilated_sparse_attention_rat_amd as rat
    B, H, T, hd = 2, 3, 300, 128
    D, W = np.array([4, 1, 16], np.int32), np.array([0, 37, 3], np.int32)
    n1, n2 = 100, 28
    T_cap = T + n1 + n2
    say(f"[checkpoint] B={B} H={H} T={T} D={list(D)} W={list(W)} {n1}+{n2} steps splits={splits}")
    inp = synth.random_case(4242 + splits, B, H, T_cap, hd, "bf16", hd ** -0.5, 3.0)
    pre = {n: np.ascontiguousarray(inp[n][:, :, :T]) for n in "qkvg"}
    c = gpu_prefill(pre, D, W, T_cap, "bf16")["cache"]
    ws = rat.decode_workspace(B, H, hd, T_cap, D, W, "cuda", num_splits=splits)
    steps = [{n: to_dev(inp[n][:, :, T + s], "bf16") for n in "qkvg"} for s in range(n1 + n2)]

    def decode(cache, s):
        x = steps[s]
        o = torch.empty_like(x["q"])
        rat.rat_decode_step(x["q"], x["k"], x["v"], x["g"], cache["state_k"], cache["state_v"],
                            cache["Kc"], cache["Vc"], cache["k_ring"], cache["v_ring"], o, D, W,
                            T + s, T_cap, num_splits=splits, workspace=ws)
        return o

    for s in range(n1):
        decode(c, s)
    torch.cuda.synchronize()
    # checkpoint: every buffer of the state, and the position, to host memory
    saved = {k: c[k].cpu().clone() for k in STATE}
    pos = T + n1

    # the uninterrupted run
    run_a = [decode(c, s) for s in range(n1, n1 + n2)]
    torch.cuda.synchronize()

    # resume: fresh buffers (filled with NaN first, so a missed copy shows),
    # the host copy restored into them
    fresh = rat.alloc_cache(B, H, hd, T_cap, D, W, torch.bfloat16, "cuda", fill=float("nan"))
    for k in STATE:
        fresh[k].copy_(saved[k].to("cuda"))
    assert pos == T + n1
    run_b = [decode(fresh, s) for s in range(n1, n1 + n2)]
    torch.cuda.synchronize()

    for i, (a, b) in enumerate(zip(run_a, run_b)):
        assert torch.equal(a, b), f"output of resumed step {pos + i} differs"
    for k in STATE:
        x, y = c[k].float(), fresh[k].float()
        assert torch.equal(torch.nan_to_num(x, nan=7.0), torch.nan_to_num(y, nan=7.0)), k

    # and the run itself matches the oracle's prefill rows
    f = {n: inp[n].astype(np.float64) for n in "qkvg"}
    ref = oracle.prefill(f["q"], f["k"], f["v"], f["g"], D, W, scale_of(hd), True)
    chk = Checks()
    chk(check_float, "o (resumed steps)", to_np(torch.stack(run_b, 2)), ref["o"][:, :, pos:T_cap],
        "bf16")
    chk.done()
