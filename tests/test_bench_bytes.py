"""The algorithmic byte counts that bench.py divides by kernel time, checked
against an enumeration of the keys each step reads (CPU only)."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("D,W,pos", [(4, 0, 300), (64, 128, 33000), (16, 5, 77), (1, 0, 10), (8, 40, 30)])
def test_decode_bytes_by_enumeration(D, W, pos):
    hd, es = 128, 2
    rows = sum(1 for j in range(pos) if oracle.in_keyset(pos, j, D, W))
    want = rows * hd * es * 2 + 4 * hd * es + hd * es + 4 * hd * 4
    want += 2 * hd * es if W > 0 else 0
    want += 2 * hd * es if pos % D == D - 1 else 0
    assert bench.decode_bytes(1, 1, hd, [D], [W], pos) == want


@pytest.mark.parametrize("D,W,pos,k", [(64, 128, 33000, 8), (4, 0, 700, 3), (16, 100, 1000, 20),
                                       (1, 0, 500, 2), (32, 0, 127, 4)])
def test_topk_decode_bytes_by_enumeration(D, W, pos, k):
    """Selected blocks: the first k eligible ones (any k blocks give the same
    count of non-anchor rows when D divides 64 or equals it)."""
    hd, es = 128, 2
    ne = max(0, pos - W) // 64
    blocks = list(range(min(k, ne)))
    extra = sum(1 for m in blocks for p in range(64 * m, 64 * m + 64) if p % D != D - 1)
    want = bench.decode_bytes(1, 1, hd, [D], [W], pos)
    want += ne * hd * 4 + extra * hd * es * 2 + 2 * hd * es
    want += hd * 4 if pos % 64 == 63 else 0
    assert bench.topk_decode_bytes(1, 1, hd, [D], [W], pos, k) == want
