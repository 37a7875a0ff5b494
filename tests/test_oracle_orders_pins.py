"""Pins for oracle/orders.py: bijection, agreement of the tile-major order with the
fractal order when a tile is one frame, cube-shaped blocks, the defining
adjacency of the Hilbert curve on a full 2^b cube, and the locality metric
ordering row-major > fractal > Hilbert/tile-major on video-like grids."""
import itertools

import numpy as np
import pytest

from oracle import fractal_positions
from oracle import orders


@pytest.mark.parametrize("T,H,W,P,N", [(4, 16, 16, 8, 64), (8, 32, 32, 4, 64), (4, 8, 8, 4, 64), (2, 8, 16, 2, 8)])
def test_tile_major_is_a_bijection_of_cubes(T, H, W, P, N):
    src = orders.tile_major_positions(T, H, W, P, N)
    assert np.array_equal(np.sort(src), np.arange(T * H * W))
    tt = N // (P * P)
    t, rem = np.divmod(src.reshape(-1, N), H * W)
    y, x = np.divmod(rem, W)
    # every block is one tt x P x P box
    for a, size in ((t, tt), (y, P), (x, P)):
        assert np.all(a.max(1) - a.min(1) == size - 1)
        assert np.all(np.min(a, 1) % size == 0)


def test_tile_major_with_one_frame_tiles_is_the_fractal_order():
    for (T, H, W, P) in [(3, 24, 40, 8), (1, 16, 16, 8), (5, 8, 24, 8)]:
        assert np.array_equal(orders.tile_major_positions(T, H, W, P, P * P), fractal_positions(T, H, W, P))


def test_tile_major_hand_case():
    # T=2, H=W=2, one 2x1x1... use tiles of 2 frames x 1 x 1 (N=2, P=1): pairs of frames per pixel
    src = orders.tile_major_positions(2, 2, 2, 1, 2)
    # pixel (0,0): tokens t=0 -> 0, t=1 -> 4; pixel (0,1): 1, 5; pixel (1,0): 2, 6; pixel (1,1): 3, 7
    assert src.tolist() == [0, 4, 1, 5, 2, 6, 3, 7]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_hilbert_walks_the_full_cube_in_unit_steps(bits):
    n = 1 << bits
    pts = np.array(list(itertools.product(range(n), repeat=3)))
    h = orders.hilbert_index_3d(pts[:, 0], pts[:, 1], pts[:, 2], bits)
    assert np.array_equal(np.sort(h), np.arange(n ** 3))          # a bijection onto 0 .. 8^bits - 1
    path = pts[np.argsort(h)]
    steps = np.abs(np.diff(path, axis=0))
    assert np.all(steps.sum(1) == 1)                               # consecutive points are face neighbours
    assert np.array_equal(path[0], [0, 0, 0])
    # the curve ends on a corner adjacent to the start corner along one axis
    end = path[-1]
    assert sorted(end.tolist()) == [0, 0, n - 1]


def test_hilbert_octants_are_contiguous():
    # every aligned 2^k sub-cube occupies one contiguous index range (self-similarity)
    bits, n = 4, 16
    pts = np.array(list(itertools.product(range(n), repeat=3)))
    h = orders.hilbert_index_3d(pts[:, 0], pts[:, 1], pts[:, 2], bits)
    for k in (1, 2, 3):
        s = 1 << k
        cell = (pts[:, 0] // s) * 10000 + (pts[:, 1] // s) * 100 + pts[:, 2] // s
        for c in np.unique(cell):
            hh = np.sort(h[cell == c])
            assert hh[-1] - hh[0] == s ** 3 - 1


@pytest.mark.parametrize("T,H,W", [(5, 24, 40), (33, 48, 80), (3, 7, 9)])
def test_hilbert_positions_bijection_on_any_grid(T, H, W):
    src = orders.hilbert_positions(T, H, W)
    assert np.array_equal(np.sort(src), np.arange(T * H * W))


def test_locality_metric_orders_the_layouts():
    T, H, W, N = 8, 32, 32, 64
    row = orders.block_spread(np.arange(T * H * W), T, H, W, N)
    frac = orders.block_spread(fractal_positions(T, H, W, 8), T, H, W, N)
    cube = orders.block_spread(orders.tile_major_positions(T, H, W, 4, N), T, H, W, N)
    hil = orders.block_spread(orders.hilbert_positions(T, H, W), T, H, W, N)
    assert row > frac > cube
    assert hil < frac
    # closed forms: a row of 32 then half a row more... row-major blocks are 2 x 32 runs
    xs = np.arange(32)
    expect_row = np.mean(np.hypot(np.concatenate([xs, xs]) - 15.5, np.repeat([-0.5, 0.5], 32)))
    assert abs(row - expect_row) < 1e-12
    # a 4 x 4 x 4 cube: mean distance of its 64 points to the centre
    g = np.arange(4) - 1.5
    d = np.sqrt(g[:, None, None] ** 2 + g[None, :, None] ** 2 + g[None, None, :] ** 2).mean()
    assert abs(cube - d) < 1e-12
