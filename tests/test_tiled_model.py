"""The pages' tile-by-tile algorithms (``oracle/tiled.py``) against the plain
definition (``oracle.c``) and against the pages' worked numbers (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import tiled

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_merge_worked_example():
    """Blocks [1,2] and [3,5]: local maxima 2 and 5; the merged maximum is 5
    and the merged sum equals the direct sum of e^[-4,-3,-2,0]."""
    g = json.load(open(os.path.join(GOLDEN, "safe_softmax_worked_example.json")))
    (b1, b2), (mx1, mx2) = g["blocks"], g["block_maxima"]
    m1, _, l1 = tiled.local_stats(np.array(b1, float))
    m2, _, l2 = tiled.local_stats(np.array(b2, float))
    assert (m1, m2) == (mx1, mx2)
    assert l1 == pytest.approx(1 + math.exp(-1), abs=1e-15)
    assert l2 == pytest.approx(1 + math.exp(-2), abs=1e-15)
    m, l = tiled.merge(m1, l1, m2, l2)
    assert m == g["merged_max"]
    direct = math.fsum(math.exp(s) for s in g["shifted"])
    assert l == pytest.approx(direct, abs=1e-15)
    assert l == pytest.approx(1.2034379904932109, abs=1e-15)
    sm, mm, ll = tiled.softmax_by_blocks(np.array(g["x"], float), 2)
    np.testing.assert_allclose(sm, scipy.special.softmax(g["x"]), rtol=0, atol=1e-16)


def test_merge_properties():
    r = np.random.default_rng(2)
    for _ in range(200):
        x = r.normal(0, 5, r.integers(2, 60))
        cut = int(r.integers(1, x.size))
        s1, s2 = tiled.local_stats(x[:cut]), tiled.local_stats(x[cut:])
        m, l = tiled.merge(s1[0], s1[2], s2[0], s2[2])
        assert m == x.max()
        assert l * math.exp(m) == pytest.approx(np.exp(x).sum(), rel=1e-13)
        # commutative
        assert tiled.merge(s2[0], s2[2], s1[0], s1[2]) == pytest.approx((m, l), rel=1e-15)
    # associative over three blocks
    x = r.normal(0, 5, 30)
    a, b, c = (tiled.local_stats(x[s:s + 10]) for s in (0, 10, 20))
    left = tiled.merge(*tiled.merge(a[0], a[2], b[0], b[2]), c[0], c[2])
    right = tiled.merge(a[0], a[2], *tiled.merge(b[0], b[2], c[0], c[2]))
    assert left == pytest.approx(right, rel=1e-14)
    # the empty state is the identity of the merge
    assert tiled.merge(-math.inf, 0.0, a[0], a[2]) == (a[0], a[2])


def test_streaming_and_blocked_softmax():
    r = np.random.default_rng(5)
    for n in (1, 5, 64, 333):
        x = r.normal(0, 4, n)
        m, l = tiled.streaming_stats(x)
        assert m == x.max()
        assert m + math.log(l) == pytest.approx(scipy.special.logsumexp(x), abs=1e-12)
        for blk in (1, 3, 16, n):
            sm, mm, ll = tiled.softmax_by_blocks(x, blk)
            np.testing.assert_allclose(sm, scipy.special.softmax(x), rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Br,Bc", [(1, 1), (2, 3), (7, 13), (16, 16), (64, 128), (101, 101)])
def test_tile_size_and_loop_order_invariance(Br, Bc, causal, oracle_lib):
    """Both loop orders, any tile sizes (non-divisors exercise ragged tails),
    with and without skipping of fully-future tiles, equal the definition."""
    r = np.random.default_rng(Br * 1000 + Bc)
    N, d = 101, 12
    Q = r.normal(0, 2, (N, d)); K = r.normal(0, 2, (N, d)); V = r.normal(0, 1, (N, d))
    O_ref, L_ref = oracle_lib.attention(Q, K, V, 0.3, causal)
    for fn in (tiled.algorithm1, tiled.q_outer):
        for skip in ((False, True) if causal else (True,)):
            O, L = fn(Q, K, V, Br, Bc, 0.3, causal, skip_future=skip)
            np.testing.assert_allclose(O, O_ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(L, L_ref, rtol=0, atol=1e-12)


def test_causal_tile_classes():
    # tile counts for square 128-tiles at N = 8192 and ragged N = 1000
    def counts(N, T):
        c = {"skip": 0, "diag": 0, "past": 0}
        for r0 in range(0, N, T):
            for c0 in range(0, N, T):
                c[tiled.causal_tile_class(r0, min(N, r0 + T), c0, min(N, c0 + T))] += 1
        return c
    assert counts(8192, 128) == {"skip": 2016, "diag": 64, "past": 2016}
    assert counts(1000, 128) == {"skip": 28, "diag": 8, "past": 28}
    # a skipped tile really is all-future, a past tile really is all-visible
    for (r0, r1, c0, c1) in [(0, 4, 4, 8), (4, 8, 0, 4), (0, 4, 3, 7), (5, 9, 5, 9)]:
        cls = tiled.causal_tile_class(r0, r1, c0, c1)
        vis = np.array([[j <= i for j in range(c0, c1)] for i in range(r0, r1)])
        assert (cls == "skip") == (not vis.any())
        assert (cls == "past") == vis.all()
