"""Pins of the oracle's Z-order permutation and block mean-pool pyramid.

Z-order: the LLSA README (page 1, reordering of non-sequential data) gives a
generator that recursively arranges the grid in quadrants (top-left,
top-right, bottom-left, bottom-right).  The oracle uses a bit-interleave closed
form instead; these tests pin it to the page's 4x4 result and to an
independent recursive quadrant construction.

Pool: the LLSA skill summary (page 2, "Core Technique" 1, hierarchical
compression) and the arXiv abstract (page 3, block-wise representation);
level l must equal the plain mean over bs^l consecutive tokens.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _quadrant_order(side):
    """Independent recursion: order[y][x] for a side x side grid."""
    if side == 1:
        return np.zeros((1, 1), np.int64)
    h = side // 2
    sub = _quadrant_order(h)
    out = np.empty((side, side), np.int64)
    cells = h * h
    out[:h, :h] = sub
    out[:h, h:] = sub + cells
    out[h:, :h] = sub + 2 * cells
    out[h:, h:] = sub + 3 * cells
    return out


def test_zorder_matches_page_4x4():
    want = np.loadtxt(os.path.join(GOLDEN, "zorder_perm_4x4.txt"), dtype=np.int64)
    got = np.array([[oracle.morton(4, y, x) for x in range(4)] for y in range(4)])
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("side", [2, 4, 8, 16, 32, 64, 128])
def test_zorder_matches_quadrant_recursion(side):
    want = _quadrant_order(side)
    got = np.array([[oracle.morton(side, y, x) for x in range(side)] for y in range(side)])
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("side", [8, 32])
def test_zorder_runs_are_square_tiles(side):
    # every run of 4^l consecutive Z positions covers one aligned 2^l x 2^l tile
    pos = np.empty(side * side, np.int64)
    for y in range(side):
        for x in range(side):
            pos[oracle.morton(side, y, x)] = y * side + x
    ys, xs = pos // side, pos % side
    for lvl in range(1, int(np.log2(side)) + 1):
        t = 2 ** lvl
        run = t * t
        for s in range(0, side * side, run):
            yy, xx = ys[s:s + run], xs[s:s + run]
            assert yy.max() - yy.min() == t - 1 and xx.max() - xx.min() == t - 1
            assert yy.min() % t == 0 and xx.min() % t == 0
            assert len(set(zip(yy.tolist(), xx.tolist()))) == run


def test_zorder_gather_and_inverse():
    rng = np.random.default_rng(1)
    side, outer, inner = 16, 3, 5
    x = rng.standard_normal((outer, side * side, inner))
    z = oracle.zorder(x, side)
    for r in [0, 1, 17, 255]:
        m = oracle.morton(side, r // side, r % side)
        np.testing.assert_array_equal(z[:, m], x[:, r])
    np.testing.assert_array_equal(oracle.zorder(z, side, inverse=True), x)
    # a permutation: the multiset of rows is unchanged
    np.testing.assert_array_equal(np.sort(z, axis=1), np.sort(x, axis=1))


@pytest.mark.parametrize("bs,L,N", [(16, 1, 256), (16, 2, 1024), (16, 3, 4096), (4, 3, 256)])
def test_pool_is_plain_mean(bs, L, N):
    rng = np.random.default_rng(2)
    G, d = 2, 7
    x = rng.standard_normal((G, N, d))
    pyr = oracle.pool(x, bs, L)
    assert len(pyr) == L
    for l in range(1, L + 1):
        n = N // bs ** l
        want = x.reshape(G, n, bs ** l, d).mean(axis=2)
        assert pyr[l - 1].shape == (G, n, d)
        np.testing.assert_allclose(pyr[l - 1], want, rtol=0, atol=1e-13)


def test_pool_block_constant_is_exact():
    rng = np.random.default_rng(3)
    G, N, d, bs, L = 1, 4096, 4, 16, 3
    # dyadic values with short mantissas, so every partial sum is exact
    coarse = np.round(rng.standard_normal((G, N // 4096, d)) * 64) / 64
    x = np.repeat(coarse, 4096, axis=1)
    for lvl in oracle.pool(x, bs, L):
        np.testing.assert_array_equal(lvl, np.repeat(coarse, lvl.shape[1], axis=1))
