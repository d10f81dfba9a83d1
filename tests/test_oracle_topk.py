"""Pins of the top-k block decode oracle (oracle/topk.py) against what is
fixed independently of it: the C oracle's decode step and key-set predicate,
brute force, and constructed selections.  CPU only."""
import numpy as np
import pytest

import oracle

HD = 32


def _case(seed, B, H, pos, std=1.0):
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s) * std
    q, k, v = r(B, H, HD), r(B, H, HD), r(B, H, HD)
    g = 1.0 / (1.0 + np.exp(-(r(B, H, HD) + 2.0)))
    sk, sv = r(B, H, HD), r(B, H, HD)
    hk, hv = r(B, H, pos, HD), r(B, H, pos, HD)
    return q, k, v, g, sk, sv, hk, hv


def _plain(args, D, W, pos, scale):
    q, k, v, g, sk, sv, hk, hv = args
    return oracle.decode_step(q, k, v, g, sk, sv, hk, hv, D, W, scale, pos, st_bf16=False)


@pytest.mark.parametrize("D,W,pos", [([4, 16], [0, 20], 300), ([3, 64], [7, 0], 257)])
def test_no_blocks_is_the_dilated_decode_step(D, W, pos):
    """k = 0 selects nothing: the step equals the C oracle's dilated decode."""
    args = _case(1, 2, 2, pos)
    D, W = np.array(D), np.array(W)
    o, sk, sv, hk, hv = _plain(args, D, W, pos, 0.3)
    r = oracle.decode_step_topk(*args, D, W, 0.3, pos, 0, st_bf16=False)
    np.testing.assert_allclose(r["o"], o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["state_k"], sk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["hat_v"], hv, rtol=1e-12, atol=1e-12)


def test_dense_heads_gain_nothing_from_blocks():
    """D = 1 makes every earlier position an anchor: any selection adds no key."""
    pos = 400
    args = _case(2, 1, 2, pos)
    D, W = np.array([1, 1]), np.array([0, 30])
    o = _plain(args, D, W, pos, 0.25)[0]
    r = oracle.decode_step_topk(*args, D, W, 0.25, pos, 5, st_bf16=False)
    assert (r["sel"] >= 0).sum() == 2 * 5
    np.testing.assert_allclose(r["o"], o, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D,W,pos", [([8, 5], [0, 64], 448), ([16, 3], [128, 0], 640)])
def test_all_blocks_make_attention_dense(D, W, pos):
    """With every eligible block selected and the window start on a block
    boundary, every earlier position is attended: the step equals dense
    causal decode (D = 1, no window) over the same history."""
    args = _case(3, 2, 2, pos)
    D, W = np.array(D), np.array(W)
    assert all((pos - w) % oracle.TOPK_BLOCK == 0 for w in W)
    dense = _plain(args, np.array([1, 1]), np.array([0, 0]), pos, 0.2)[0]
    r = oracle.decode_step_topk(*args, D, W, 0.2, pos, 10 ** 6, st_bf16=False)
    np.testing.assert_allclose(r["o"], dense, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D,W,pos", [(4, 0, 300), (5, 37, 517), (64, 128, 1000), (2, 200, 260)])
def test_key_set_is_the_union_by_definition(D, W, pos):
    """Attended positions = the C oracle's dilated key set (minus the own
    position) united with the selected blocks' positions, each once."""
    rng = np.random.default_rng(pos)
    n_elig = max(0, pos - W) // oracle.TOPK_BLOCK
    blocks = sorted(rng.choice(n_elig, size=min(3, n_elig), replace=False).tolist()) if n_elig else []
    keys = oracle.keys_topk(pos, D, W, blocks)
    assert len(keys) == len(set(keys))
    want = {j for j in range(pos) if oracle.in_keyset(pos, j, D, W)}
    for m in blocks:
        want |= set(range(64 * m, 64 * m + 64))
    assert set(keys) == want


def test_selection_brute_force_and_ties():
    """The top-k are the highest block-mean scores; equal scores go to the
    lower block; blocks that reach into the window are never candidates."""
    pos, W = 64 * 10 + 5, 70
    q = np.zeros((1, 1, HD))
    q[0, 0, 0] = 1.0
    hk = np.zeros((1, 1, pos, HD))
    # block means along channel 0: block 7 best, blocks 2 and 5 tie, block 9
    # (inside the window's reach) would be best of all
    for m, val in [(7, 5.0), (2, 3.0), (5, 3.0), (9, 9.0), (0, -1.0)]:
        hk[0, 0, 64 * m:64 * m + 64, 0] = val
    n_elig = max(0, pos - W) // 64
    assert n_elig == 8  # blocks 0..7
    sel = oracle.select_blocks(q[0, 0], oracle.block_means(hk)[0, 0], n_elig, 3)
    assert sel.tolist() == [7, 2, 5]
    # brute force over every 3-subset: the selection maximises the score sum
    sc = oracle.block_means(hk)[0, 0, :n_elig] @ q[0, 0]
    import itertools
    best = max(sum(sc[list(c)]) for c in itertools.combinations(range(n_elig), 3))
    assert sum(sc[sel]) == best


def test_block_means_by_loop():
    hk = np.random.default_rng(4).standard_normal((1, 2, 200, 8))
    m = oracle.block_means(hk)
    assert m.shape == (1, 2, 3, 8)
    for h in range(2):
        for b in range(3):
            ref = sum(hk[0, h, 64 * b + i] for i in range(64)) / 64.0
            np.testing.assert_allclose(m[0, h, b], ref, rtol=1e-13)


def test_given_selection_is_used():
    """An explicit selection (e.g. a GPU's) replaces the oracle's own."""
    pos = 520
    args = _case(5, 1, 1, pos)
    D, W = np.array([8]), np.array([0])
    own = oracle.decode_step_topk(*args, D, W, 0.3, pos, 2, st_bf16=False)
    other = np.array([[[0, 1]]]) if own["sel"][0, 0].tolist() != [0, 1] else np.array([[[2, 3]]])
    r = oracle.decode_step_topk(*args, D, W, 0.3, pos, 2, st_bf16=False, sel=other)
    assert r["sel"].tolist() == other.tolist()
    assert not np.allclose(r["o"], own["o"])
