"""The library's host-side order tables (bsa_order_table) against the oracle's
(oracle/orders.py), integer for integer; needs no GPU."""
import numpy as np
import pytest

import oracle
from oracle import orders

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")


@pytest.fixture(scope="module", autouse=True)
def _lib_built():
    import os
    if not os.path.exists(bsa.LIB_PATH):
        pytest.skip("libbsa.so not built")


GRIDS = [(4, 16, 16, 8), (3, 24, 40, 8), (21, 32, 48, 8), (33, 48, 80, 8), (8, 32, 32, 4), (4, 8, 8, 4), (12, 16, 40, 4)]


@pytest.mark.parametrize("T,H,W,P", [g for g in GRIDS if g[3] * g[3] == 64])   # N = 64 = P*P
def test_fractal_table(T, H, W, P):
    got = bsa.order_table(bsa.VideoGrid(T, H, W, P, 64), "fractal").numpy()
    assert np.array_equal(got, oracle.fractal_positions(T, H, W, P))


@pytest.mark.parametrize("T,H,W,P", GRIDS)
def test_tile_major_table(T, H, W, P):
    g = bsa.VideoGrid(T, H, W, P, 64)
    if T % (64 // (P * P)):
        with pytest.raises(bsa.BSAError):
            bsa.order_table(g, "tile_major")
        return
    got = bsa.order_table(g, "tile_major").numpy()
    assert np.array_equal(got, orders.tile_major_positions(T, H, W, P, 64))


@pytest.mark.parametrize("T,H,W,P", GRIDS)
def test_hilbert_table(T, H, W, P):
    got = bsa.order_table(bsa.VideoGrid(T, H, W, P, 64), "hilbert").numpy()
    assert np.array_equal(got, orders.hilbert_positions(T, H, W))


def test_unknown_order_is_rejected():
    with pytest.raises(ValueError):
        bsa.order_table(bsa.VideoGrid(4, 16, 16), "zorder")
    import ctypes
    from block_sparse_attention_fractal_amd import _lib
    p = _lib.Problem(1, 1, 4, 16, 16, 128, 8, 64, 1, 0)
    table = (ctypes.c_int32 * (4 * 16 * 16))()
    assert _lib.lib().bsa_order_table(ctypes.byref(p), 7, table) == 1


def test_locality_of_the_orders_on_video_grids():
    """Block locality (mean token distance to the block centroid, oracle metric) of
    the library's tables: the Hilbert and tile-major orders are tighter than the
    fractal order, which is tighter than row-major."""
    T, H, W = 8, 32, 32
    spread = {name: orders.block_spread(bsa.order_table(bsa.VideoGrid(T, H, W, 8 if name == "fractal" else 4, 64),
                                                        name).numpy(), T, H, W, 64)
              for name in ("fractal", "tile_major", "hilbert")}
    row = orders.block_spread(np.arange(T * H * W), T, H, W, 64)
    assert row > spread["fractal"] > spread["tile_major"]
    assert spread["hilbert"] < spread["fractal"]
