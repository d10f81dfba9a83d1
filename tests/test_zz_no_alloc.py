"""rat_decode_step_noalloc: the decode step with its split-K partials in the
library's own device array instead of a caller workspace.  Through the C ABI
it must give exactly what rat_decode_step gives with a workspace (same
kernels, same split choice): two calls in a row on one device, the second
with a smaller batch, so the second reuses the array the first left behind.
Both are also held to the oracle's prefill rows at the bf16 tolerance."""
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

CASES = [
    # B, H, T, D, W, splits, steps
    (2, 4, 700, [4, 1, 16, 8], [0, 37, 3, 0], 4, 3),
    (1, 3, 300, [2, 5, 1], [9, 0, 0], 3, 2),      # smaller, after the first
]

STATE = ("state_k", "state_v", "Kc", "Vc", "k_ring", "v_ring")


def test_noalloc_decode_equals_workspace_decode_twice():
    import dilated_sparse_attention_rat_amd as rat
    hd = 128
    chk = Checks()
    for i, (B, H, T, D, W, splits, steps) in enumerate(CASES):
        D, W = np.array(D, np.int32), np.array(W, np.int32)
        T_cap = T + steps
        say(f"[noalloc] call {i}: B={B} H={H} T={T} D={list(D)} W={list(W)} splits={splits}")
        assert B * H * splits * (hd + 2) * 4 <= rat.binding.NOALLOC_SCRATCH_BYTES
        inp = synth.random_case(900 + i, B, H, T_cap, hd, "bf16", hd ** -0.5, 3.0)
        pre = {n: np.ascontiguousarray(inp[n][:, :, :T]) for n in "qkvg"}
        ca = gpu_prefill(pre, D, W, T_cap, "bf16")["cache"]
        cb = gpu_prefill(pre, D, W, T_cap, "bf16")["cache"]
        ws = rat.decode_workspace(B, H, hd, T_cap, D, W, "cuda", num_splits=splits)
        oa, ob = [], []
        for s in range(steps):
            x = {n: to_dev(inp[n][:, :, T + s], "bf16") for n in "qkvg"}
            o1, o2 = torch.empty_like(x["q"]), torch.empty_like(x["q"])
            rat.rat_decode_step(x["q"], x["k"], x["v"], x["g"], ca["state_k"], ca["state_v"],
                                ca["Kc"], ca["Vc"], ca["k_ring"], ca["v_ring"], o1, D, W, T + s,
                                T_cap, num_splits=splits, workspace=ws)
            rat.rat_decode_step_noalloc(x["q"], x["k"], x["v"], x["g"], cb["state_k"],
                                        cb["state_v"], cb["Kc"], cb["Vc"], cb["k_ring"],
                                        cb["v_ring"], o2, D, W, T + s, T_cap, num_splits=splits)
            oa.append(o1)
            ob.append(o2)
        torch.cuda.synchronize()
        for s in range(steps):
            assert torch.equal(oa[s], ob[s]), f"call {i}: output of step {T + s} differs"
        for k in STATE:
            x, y = ca[k].float(), cb[k].float()
            assert torch.equal(torch.nan_to_num(x, nan=7.0), torch.nan_to_num(y, nan=7.0)), k
        f = {n: inp[n].astype(np.float64) for n in "qkvg"}
        ref = oracle.prefill(f["q"], f["k"], f["v"], f["g"], D, W, scale_of(hd), True)
        chk(check_float, f"o (call {i})", to_np(torch.stack(ob, 2)), ref["o"][:, :, T:T_cap],
            "bf16")
    chk.done()
