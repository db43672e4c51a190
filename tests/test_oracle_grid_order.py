"""Pins of the oracle's grid order: the quadtree order of the LLSA README
(page 1, reordering of non-sequential data such as images or videos)
extended to rectangles whose sides are not powers of two and, as an octree,
to video.

The rule: cut the grid into the largest power-of-two squares (cubes when there
are several frames) that divide every side, take the tiles in raster order and
the cells of a tile in quadtree (octree) order -- top before bottom before
left/right at every scale, and an earlier frame half before a later one.  The
oracle computes it with a bit-interleave closed form; the tests build the same
order by independent recursion over quadrants and octants, and check the
locality that makes the order useful: aligned runs of 16 tokens are 4 x 4
patches (2 x 2 x 4 boxes in video), runs of 8 are 2 x 2 x 2 cubes.
"""
import numpy as np
import pytest

import oracle


def _quadrant_order(side):
    """order[y][x] of a side x side tile by recursion over quadrants."""
    if side == 1:
        return np.zeros((1, 1), np.int64)
    h = side // 2
    sub = _quadrant_order(h)
    cells = h * h
    out = np.empty((side, side), np.int64)
    out[:h, :h] = sub
    out[:h, h:] = sub + cells
    out[h:, :h] = sub + 2 * cells
    out[h:, h:] = sub + 3 * cells
    return out


def _octant_order(side):
    """order[t][y][x] of a side^3 cube by recursion over octants: the earlier
    frame half first, then the top half, then the left half."""
    if side == 1:
        return np.zeros((1, 1, 1), np.int64)
    h = side // 2
    sub = _octant_order(h)
    cells = h ** 3
    out = np.empty((side, side, side), np.int64)
    for tb in (0, 1):
        for yb in (0, 1):
            for xb in (0, 1):
                out[tb * h:(tb + 1) * h, yb * h:(yb + 1) * h, xb * h:(xb + 1) * h] = \
                    sub + (4 * tb + 2 * yb + xb) * cells
    return out


def _pow2_part(n):
    return n & -n


def _expected(T, H, W):
    """order[t][y][x] built tile by tile from the recursive constructions."""
    S = min(_pow2_part(H), _pow2_part(W))
    if T > 1:
        S = min(S, _pow2_part(T))
        tile = _octant_order(S)
    else:
        tile = _quadrant_order(S)[None]
    cells = tile.size
    out = np.empty((T, H, W), np.int64)
    st = S if T > 1 else 1
    k = 0
    for t0 in range(0, T, st):
        for y0 in range(0, H, S):
            for x0 in range(0, W, S):
                out[t0:t0 + st, y0:y0 + S, x0:x0 + S] = tile + k * cells
                k += 1
    return out


def _got(T, H, W):
    return np.array([[[oracle.grid_index(T, H, W, t, y, x) for x in range(W)]
                      for y in range(H)] for t in range(T)])


@pytest.mark.parametrize("side", [1, 2, 4, 16, 64])
def test_square_image_is_the_quadtree_order(side):
    got = _got(1, side, side)[0]
    np.testing.assert_array_equal(got, _quadrant_order(side))
    np.testing.assert_array_equal(
        got, [[oracle.morton(side, y, x) for x in range(side)] for y in range(side)])


@pytest.mark.parametrize("T,H,W", [
    (1, 2, 4), (1, 4, 16), (1, 16, 4), (1, 32, 8),     # power-of-two rectangles
    (1, 48, 80), (1, 12, 20), (1, 3, 5), (1, 24, 16),   # other sides
    (2, 2, 2), (4, 8, 8), (2, 8, 16), (8, 4, 4),        # video, power-of-two sides
    (3, 8, 8), (6, 12, 20), (4, 48, 32),                # video, other sides
])
def test_grid_order_matches_recursive_construction(T, H, W):
    np.testing.assert_array_equal(_got(T, H, W), _expected(T, H, W))


def test_two_by_four_image_by_hand():
    # two 2x2 tiles side by side, each in quadtree order
    order = [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3)]
    for pos, (y, x) in enumerate(order):
        assert oracle.grid_index(1, 2, 4, 0, y, x) == pos


def test_one_cube_by_hand():
    for t in (0, 1):
        for y in (0, 1):
            for x in (0, 1):
                assert oracle.grid_index(2, 2, 2, t, y, x) == 4 * t + 2 * y + x


@pytest.mark.parametrize("T,H,W", [(1, 48, 80), (1, 64, 16), (4, 32, 32), (8, 16, 24)])
def test_aligned_runs_are_compact_boxes(T, H, W):
    n = T * H * W
    cells = np.empty((n, 3), np.int64)
    for t in range(T):
        for y in range(H):
            for x in range(W):
                cells[oracle.grid_index(T, H, W, t, y, x)] = (t, y, x)
    assert len({tuple(c) for c in cells.tolist()}) == n  # a permutation
    # image: 16 = one 4x4 patch; video: 8 = one 2x2x2 cube, 16 = 2x2x4 (t, y, x)
    shapes = {16: (1, 4, 4)} if T == 1 else {8: (2, 2, 2), 16: (2, 2, 4), 64: (4, 4, 4)}
    for run, shape in shapes.items():
        for s in range(0, n, run):
            c = cells[s:s + run]
            ext = tuple(int(v) for v in c.max(0) - c.min(0) + 1)
            assert ext == shape
            assert all(c.min(0)[a] % shape[a] == 0 for a in range(3))


def test_grid_gather_and_inverse():
    rng = np.random.default_rng(3)
    T, H, W, outer, inner = 2, 8, 12, 3, 5
    n = T * H * W
    x = rng.standard_normal((outer, n, inner))
    z = oracle.grid_order(x, T, H, W)
    for r in (0, 1, 13, n - 1):
        t, y, xx = r // (H * W), (r // W) % H, r % W
        np.testing.assert_array_equal(z[:, oracle.grid_index(T, H, W, t, y, xx)], x[:, r])
    np.testing.assert_array_equal(oracle.grid_order(z, T, H, W, inverse=True), x)


def test_single_frame_grid_order_equals_square_zorder():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 32 * 32, 3))
    np.testing.assert_array_equal(oracle.grid_order(x, 1, 32, 32), oracle.zorder(x, 32))
