"""Decode step of dilated attention combined with top-k block selection
(plain numpy, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Method: RAT+ abstract (v1) -- a RAT+ model sparsified to top-k block
attention beats plain attention sparsified the same way; zhichai.net deep
dive "RAT+ 深度拆解", section 四 -- dilation and top-k block selection
combine: the dilated anchors cover the whole past, the selected blocks add
density where the query needs it.  The pages give no block size, scoring
rule or k; this oracle takes the following reading of them:

  * blocks are the aligned runs of TOPK_BLOCK positions [64m, 64m+63];
  * a block is eligible for the query at position t when it lies entirely
    before the window start: 64m + 63 < max(0, t - W);
  * its score is q_t . kbar_m, kbar_m the mean of the stored key states of
    its positions; the k highest scores are selected (equal scores: the
    lower block index first; every eligible block when there are at most k);
  * the query attends to its dilated key set (anchors a < floor(max(0,
    t-W)/D), window t-W .. t-1, its own position) and to every position of
    the selected blocks that is not already an anchor -- an anchor position
    inside an eligible block is always an included anchor, so the union
    counts it once.
"""
from __future__ import annotations

import numpy as np

from .oracle import round_bf16

TOPK_BLOCK = 64


def block_means(hk_hist) -> np.ndarray:
    """Mean key state of every complete block: [B,H,T,hd] -> [B,H,T//64,hd]."""
    hk = np.asarray(hk_hist, dtype=np.float64)
    B, H, T, hd = hk.shape
    n = T // TOPK_BLOCK
    return hk[:, :, :n * TOPK_BLOCK].reshape(B, H, n, TOPK_BLOCK, hd).mean(axis=3)


def select_blocks(q, means, n_elig: int, k_sel: int) -> np.ndarray:
    """Indices of the k best eligible blocks for one query, best first
    (equal scores: lower index first)."""
    scores = means[:n_elig] @ q
    order = sorted(range(n_elig), key=lambda m: (-scores[m], m))
    return np.array(order[:min(k_sel, n_elig)], dtype=np.int64)


def keys_topk(t: int, D: int, W: int, blocks) -> list:
    """Positions the query at t attends to besides itself: anchors, window,
    then the selected blocks' positions that are not anchors (in that order;
    the three parts are disjoint)."""
    lo = max(0, t - W)
    keys = [a * D + D - 1 for a in range(lo // D)]
    keys += list(range(lo, t))
    for m in blocks:
        assert TOPK_BLOCK * m + TOPK_BLOCK - 1 < lo, "block not eligible"
        keys += [p for p in range(TOPK_BLOCK * m, TOPK_BLOCK * m + TOPK_BLOCK) if p % D != D - 1]
    return keys


def decode_step_topk(q, k, v, g, state_k, state_v, hk_hist, hv_hist, D, W, scale, pos: int,
                     k_sel: int, st_bf16: bool, sel=None):
    """One decode step at position pos with top-k block selection.

    q, k, v, g: [B,H,hd]; state_k/v: [B,H,hd] (not modified); hk_hist,
    hv_hist: [B,H,pos,hd] stored states of the positions before pos.
    sel: optional [B,H,k_sel] block indices to use instead of the oracle's
    own selection (entries < 0 ignored) -- for checking an output computed
    from a selection made in another precision.
    Returns dict(o, state_k, state_v, hat_k, hat_v, sel, scores, n_elig)."""
    q, k, v, g = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g))
    sk = np.asarray(state_k, dtype=np.float64)
    sv = np.asarray(state_v, dtype=np.float64)
    hk = np.asarray(hk_hist, dtype=np.float64)
    hv = np.asarray(hv_hist, dtype=np.float64)
    B, H, hd = q.shape
    assert hk.shape == (B, H, pos, hd) and hv.shape == (B, H, pos, hd)
    # the recurrence, one state update (deep dive, section 2.1)
    nsk = g * sk + (1.0 - g) * k
    nsv = g * sv + (1.0 - g) * v
    hat_k = round_bf16(nsk) if st_bf16 else nsk
    hat_v = round_bf16(nsv) if st_bf16 else nsv
    means = block_means(hk)
    o = np.empty((B, H, hd))
    used = np.full((B, H, k_sel), -1, dtype=np.int64)
    scores_all = {}
    n_elig = np.zeros((B, H), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            Dh, Wh = int(D[h]), int(W[h])
            ne = max(0, pos - Wh) // TOPK_BLOCK
            n_elig[b, h] = ne
            scores_all[(b, h)] = means[b, h, :ne] @ q[b, h]
            if sel is None:
                blocks = select_blocks(q[b, h], means[b, h], ne, k_sel)
            else:
                blocks = np.array([m for m in np.asarray(sel)[b, h] if m >= 0], dtype=np.int64)
            used[b, h, :len(blocks)] = blocks
            keys = keys_topk(pos, Dh, Wh, blocks)
            K = np.concatenate([hk[b, h, keys], hat_k[b, h][None]], axis=0)
            V = np.concatenate([hv[b, h, keys], hat_v[b, h][None]], axis=0)
            logit = scale * (K @ q[b, h])
            w = np.exp(logit - logit.max())
            o[b, h] = (w / w.sum()) @ V
    return dict(o=o, state_k=nsk, state_v=nsv, hat_k=hat_k, hat_v=hat_v, sel=used,
                scores=scores_all, n_elig=n_elig)
