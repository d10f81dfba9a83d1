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


@pytest.mark.parametrize("W", [0, 1, 37, 64, 100, 129])
def test_eligible_blocks_by_enumeration(W):
    """The number of eligible blocks, and the selection with k above it, equal
    an enumeration of the blocks that end before the window start."""
    for pos in [0, 1, 63, 64, 65, 127, 128, 129, 200, 300]:
        args = _case(6, 1, 1, pos)
        r = oracle.decode_step_topk(*args, np.array([3]), np.array([W]), 0.3, pos, 100,
                                    st_bf16=False)
        want = [m for m in range(pos // 64 + 1) if 64 * m + 63 < max(0, pos - W)]
        assert int(r["n_elig"][0, 0]) == len(want)
        assert sorted(int(m) for m in r["sel"][0, 0] if m >= 0) == want


def _all_pins():
    test_no_blocks_is_the_dilated_decode_step([4, 16], [0, 20], 300)
    test_no_blocks_is_the_dilated_decode_step([3, 64], [7, 0], 257)
    test_dense_heads_gain_nothing_from_blocks()
    test_all_blocks_make_attention_dense([8, 5], [0, 64], 448)
    for D, W, pos in [(4, 0, 300), (5, 37, 517), (64, 128, 1000), (2, 200, 260)]:
        test_key_set_is_the_union_by_definition(D, W, pos)
    test_selection_brute_force_and_ties()
    test_block_means_by_loop()
    test_given_selection_is_used()
    for W in [0, 37, 100]:
        test_eligible_blocks_by_enumeration(W)


# planted mistakes in a copy of oracle/topk.py: some pin above must fail
TOPK_MUTANTS = [
    ("eligibility ignores the window", "ne = max(0, pos - Wh) // TOPK_BLOCK",
     "ne = pos // TOPK_BLOCK"),
    ("ties go to the higher block", "key=lambda m: (-scores[m], m)", "key=lambda m: (-scores[m], -m)"),
    ("lowest scores selected", "key=lambda m: (-scores[m], m)", "key=lambda m: (scores[m], m)"),
    ("anchors counted twice", "if p % D != D - 1]", "]"),
    ("window dropped from the key set", "keys += list(range(lo, t))", "keys += []"),
    ("block mean over 63 rows", ".mean(axis=3)", "[:, :, :, :63].mean(axis=3)"),
    ("own position dropped",
     "K = np.concatenate([hk[b, h, keys], hat_k[b, h][None]], axis=0)\n"
     "            V = np.concatenate([hv[b, h, keys], hat_v[b, h][None]], axis=0)",
     "K = hk[b, h, keys]\n            V = hv[b, h, keys]"),
    ("scale dropped", "logit = scale * (K @ q[b, h])", "logit = K @ q[b, h]"),
    ("gate roles swapped", "nsk = g * sk + (1.0 - g) * k", "nsk = (1.0 - g) * sk + g * k"),
    ("given selection ignored", "if sel is None:", "if True:"),
]


@pytest.mark.parametrize("desc,orig,mut", TOPK_MUTANTS, ids=[m[0] for m in TOPK_MUTANTS])
def test_planted_topk_mistake_is_caught(monkeypatch, desc, orig, mut):
    import types
    import oracle.topk as tk
    src = open(tk.__file__).read()
    assert src.count(orig) == 1, desc
    mod = types.ModuleType("oracle.topk_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(orig, mut), tk.__file__, "exec"), mod.__dict__)
    for name in ("decode_step_topk", "select_blocks", "keys_topk", "block_means"):
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    with pytest.raises(AssertionError):
        _all_pins()
