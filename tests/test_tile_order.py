"""The persistent-grid tile order (tkg_tile_order, the code the kernels run):
every launch form visits every output tile exactly once, and the XCD-block
order gives each XCD a compact block per round. Host logic, no GPU."""
import ctypes

import pytest

import tiled_dense_gemm_amd as tkg


def _order(tiles_m, tiles_n, grid, remap, group_m):
    return [tkg.tile_order(t, grid, remap, tiles_m, tiles_n, group_m)
            for t in range(tiles_m * tiles_n)]


SHAPES = [
    # (tiles_m, tiles_n, grid, group_m): full bands, a partial last band,
    # grids below, at and above the tile count, group_m not dividing grid
    # (group_m at most tiles_m, as the planner clamps it)
    (32, 32, 256, 8), (32, 32, 256, 16), (64, 64, 256, 16), (64, 64, 256, 32),
    (24, 40, 256, 8), (30, 17, 256, 8), (7, 9, 256, 7), (5, 3, 16, 5),
    (32, 56, 256, 8), (16, 16, 40, 3), (33, 31, 64, 4), (8, 8, 512, 8),
]


@pytest.mark.parametrize("tiles_m,tiles_n,grid,group_m", SHAPES)
@pytest.mark.parametrize("remap", [0, 1, 2])
def test_every_tile_once(tiles_m, tiles_n, grid, group_m, remap):
    got = _order(tiles_m, tiles_n, grid, remap, group_m)
    assert sorted(got) == [(i, j) for i in range(tiles_m) for j in range(tiles_n)]


@pytest.mark.parametrize("tiles_m,tiles_n,grid,group_m",
                         [(32, 32, 256, 8), (64, 64, 256, 16), (64, 64, 256, 32),
                          (32, 64, 256, 32)])
def test_xcd_blocks_are_rectangles(tiles_m, tiles_n, grid, group_m):
    # remap 2 on full-band rounds: the grid/8 tiles one XCD runs at the same
    # time (virtual ids x*grid/8 .. +grid/8-1 of a round) form an h x w block
    # with h + w as small as the band's rectangle allows
    order = _order(tiles_m, tiles_n, grid, 2, group_m)
    per = grid // 8
    cols = grid // group_m
    best = min(group_m // (8 // b) + cols // b for b in (8, 4, 2, 1)
               if group_m % (8 // b) == 0 and cols % b == 0)
    for r0 in range(0, tiles_m * tiles_n, grid):
        for x in range(8):
            blk = order[r0 + x * per: r0 + (x + 1) * per]
            rows = {p for p, _ in blk}
            cols_ = {q for _, q in blk}
            assert len(rows) * len(cols_) == per, (r0, x, blk)
            assert max(rows) - min(rows) + 1 == len(rows)
            assert max(cols_) - min(cols_) + 1 == len(cols_)
            assert len(rows) + len(cols_) == best


@pytest.mark.parametrize("M,N,K", [(6144, 6144, 4096), (4096, 5120, 4096),
                                   (8192, 9216, 2048), (2816, 8192, 4096)])
@pytest.mark.parametrize("dtype", [tkg.DTYPE_BF16, tkg.DTYPE_FP8])
def test_two_launch_products_cover_every_quadrant_once(M, N, K, dtype):
    # the first launch runs items t < units (whole 256 x 256 tiles), the
    # tail launch the remaining tiles' 128 x 128 quadrants: together every
    # quadrant of the output exactly once
    p = tkg.plan_launch(dtype, M, N, K)
    tm, tn = M // 256, N // 256
    if p["tail_units"] == 0:
        pytest.skip("no tail launch for this shape")
    seen = []
    for t in range(p["units"]):
        i, j = tkg.tile_order(t, p["grid"], p["xcd_remap"], tm, tn, p["group_m"])
        seen += [(2 * i + a, 2 * j + b) for a in (0, 1) for b in (0, 1)]
    for u in range(p["tail_units"]):
        seen.append(tkg.tile_order(u, p["grid"], p["xcd_remap"], tm, tn, p["group_m"],
                                   quad_base=p["units"]))
    assert sorted(seen) == [(i, j) for i in range(2 * tm) for j in range(2 * tn)]


def test_tile_order_argument_errors():
    bad = tkg.STATUS["TKG_ERR_SHAPE"]
    for args in [(0, 0, 1, 4, 4, 2, -1), (0, 8, 3, 4, 4, 2, -1), (0, 8, 1, 0, 4, 2, -1),
                 (0, 8, 1, 4, 4, 0, -1), (16, 8, 1, 4, 4, 2, -1), (-1, 8, 1, 4, 4, 2, -1),
                 (4, 8, 1, 4, 4, 2, 15), (0, 8, 1, 4, 4, 2, 17), (0, 8, 1, 4, 4, 5, -1)]:
        pm, pn = ctypes.c_int32(), ctypes.c_int32()
        assert tkg.lib.tkg_tile_order(*args, ctypes.byref(pm), ctypes.byref(pn)) == bad, args
    assert tkg.lib.tkg_tile_order(0, 8, 1, 4, 4, 2, -1, None, None) == tkg.STATUS["TKG_ERR_NULL"]
