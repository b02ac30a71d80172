"""The LDS bank model: pinned to the page's printed H100 results, then used
to show that every fragment read the kernels issue is conflict-free under
both candidate gfx950 geometries."""
import json
import os

import pytest

from tiled_dense_gemm_amd import lds_bank_model as bm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bank_model_page1.json")


def test_page_model_reproduces_printed_degrees():
    g = json.load(open(GOLDEN))
    assert bm.page_model(g["row_stride_bytes"]) == g["naive_row_major_degree"]
    assert bm.page_model(g["row_stride_bytes"], bm.page_swizzle) == g["swizzle_128B_degree"]


def test_page_swizzles_are_bijections():
    # Each of the 32/64/128-byte swizzles permutes the 16-byte chunks of
    # every aligned span of span*8 bytes (page "ThunderKittens: Simple, Fast,
    # and Adorable AI Kernels", section 3.4, "Shared Memory Tiles").
    for span in (32, 64, 128):
        size = span * 8
        for base in (0, size, 5 * size):
            img = {bm.page_swizzle(base + a, span) for a in range(0, size, 16)}
            assert img == set(range(base, base + size, 16))


def test_model_detects_conflicts():
    # negative control: 16 lanes reading the same bank column
    addrs = [r * 256 for r in range(64)]
    assert bm.conflict_degree(addrs, 16, 64, 16) == 16
    assert bm.conflict_degree(addrs, 16, 32, 8) == 8
    # broadcast of one word is not a conflict
    assert bm.conflict_degree([0] * 64, 4, 32, 32) == 1


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("geom", sorted(bm.GFX950_GEOMETRIES))
def test_kernel_fragment_reads_conflict_free(dtype, geom):
    banks, lanes = bm.GFX950_GEOMETRIES[geom]
    pats = bm.kernel_fragment_reads(dtype)
    assert pats
    assert bm.worst_degree(pats, 16, banks, lanes) == 1


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_unswizzled_layout_would_conflict(dtype):
    # the same reads without the XOR (row * row_bytes + chunk * 16)
    import tiled_dense_gemm_amd as tkg
    rb = tkg.lds_row_bytes(dtype)
    pats = bm.kernel_fragment_reads(dtype)
    # logical chunks: all lanes of a half read the same logical chunk
    unsw = []
    for p in pats:
        rows = [a // rb for a in p]
        # chunk each half reads before swizzling = the one row 0 reads (mask 0)
        c0 = (p[0] % rb) // 16
        c1 = (p[32] % rb) // 16
        unsw.append([rows[l] * rb + 16 * (c0 if l < 32 else c1) for l in range(64)])
    for geom, (banks, lanes) in bm.GFX950_GEOMETRIES.items():
        assert bm.worst_degree(unsw, 16, banks, lanes) > 1, geom


def test_swizzle_permutes_chunks_of_each_row():
    import tiled_dense_gemm_amd as tkg
    for dtype in (0, 1, 2):
        rb = tkg.lds_row_bytes(dtype)
        pats = bm.kernel_fragment_reads(dtype)
        seen = {}
        for p in pats:
            for a in p:
                seen.setdefault(a // rb, set()).add(a % rb)
        for row, offs in seen.items():
            assert offs == set(range(0, rb, 16)), (dtype, row)


def test_fp4_scale_reads():
    # 8-byte reads of consecutive 8-byte rows: conflict-free in both
    # geometries (lanes 32..63 repeat the rows of lanes 0..31)
    addrs = bm.scale_read_pattern(8, 8)
    for banks, _ in bm.GFX950_GEOMETRIES.values():
        assert bm.conflict_degree(addrs, 8, banks, bm.phase_lanes(8, banks)) == 1
