"""LDS bank conflicts: the page's printed H100 model, and the MI355X
measurements that choose and check the kernels' swizzled layouts.

The gfx950 table (tests/golden/lds_probe_gfx950.json) was measured with
tiled_dense_gemm_amd/probes/lds_bank_probe.hip and rocprofv3's
SQ_LDS_BANK_CONFLICT counter (profiles/lds_bank_probe_gfx950.md gives the
command); every fragment read the library reports must appear in it,
address for address, as conflict-free."""
import json
import os

import pytest

import tiled_dense_gemm_amd as tkg
from tiled_dense_gemm_amd import lds_bank_model as bm

GOLD = os.path.join(os.path.dirname(__file__), "golden")
PAGE = json.load(open(os.path.join(GOLD, "bank_model_page1.json")))
PROBE = json.load(open(os.path.join(GOLD, "lds_probe_gfx950.json")))
MEASURED = {(p["bytes"], tuple(p["addresses"])): p for p in PROBE["patterns"]}


def measured(addrs, nbytes=16):
    return MEASURED.get((nbytes, tuple(addrs)))


def by_name(name):
    return next(p for p in PROBE["patterns"] if p["name"] == name)


def test_page_model_reproduces_printed_degrees():
    assert bm.page_model(PAGE["row_stride_bytes"]) == PAGE["naive_row_major_degree"]
    assert bm.page_model(PAGE["row_stride_bytes"], bm.page_swizzle) == PAGE["swizzle_128B_degree"]


def test_page_swizzles_are_bijections():
    # Each of the 32/64/128-byte swizzles permutes the 16-byte chunks of
    # every aligned span of span*8 bytes (page "ThunderKittens: Simple, Fast,
    # and Adorable AI Kernels", section 3.4, "Shared Memory Tiles").
    for span in (32, 64, 128):
        size = span * 8
        for base in (0, size, 5 * size):
            img = {bm.page_swizzle(base + a, span) for a in range(0, size, 16)}
            assert img == set(range(base, base + size, 16))


def test_measured_phase_geometry():
    # ds_read_b128 serves 16 consecutive lanes per phase (lanes l and l^1..8
    # collide in one bank group, l^16 and l^32 do not); b64 and b32 serve 32
    for w, phase in ((128, 16), (64, 32), (32, 32)):
        assert by_name("b%d contiguous" % w)["degree"] == 1
        for d in (1, 2, 4, 8, 16, 32):
            deg = by_name("b%d lanes l and l^%d share a bank group" % (w, d))["degree"]
            assert deg == (2 if d < phase else 1), (w, d, deg)


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_kernel_fragment_reads_measured_conflict_free(dtype):
    pats = bm.kernel_fragment_reads(dtype)
    assert pats
    for p in pats:
        m = measured(p)
        assert m is not None, "fragment read pattern not in the measured table"
        assert " swizzled " in m["name"] and m["degree"] == 1, m["name"]


def test_unswizzled_reads_measured_conflicting():
    un = [p for p in PROBE["patterns"] if " unswizzled " in p["name"]]
    assert len(un) == 80
    assert all(p["degree"] >= 4 for p in un)


def _linear_index(mask_of_row):
    # A (3x4 over GF(2)) with mask(r) = A * bits(r) for r < 16, as the probe
    # enumerates it: row b of A is bits 4b..4b+3 of the index
    for A in range(4096):
        ok = True
        for r in range(16):
            m = 0
            for b in range(3):
                m |= (bin(((A >> (4 * b)) & 15) & r).count("1") & 1) << b
            if m != mask_of_row(r):
                ok = False
                break
        if ok:
            return A
    return None


def test_swizzle_choice_is_measured_conflict_free():
    # the 128-byte-row swizzle of the library (read back from the first 16
    # rows of a fragment) against the search over all linear swizzles
    p = tkg.lds_fragment_offsets(tkg.DTYPE_BF16, 0, 0, 0)
    mask = {(a // 128): ((a % 128) // 16) ^ (l // 16) for l, a in enumerate(p)}
    A = _linear_index(lambda r: mask[r])
    search = PROBE["search_16x16_degrees"]
    assert A is not None and search[A] == 1
    # the XOR with row bit 3 alone, chunk ^ (r & 7) ^ ((r >> 3) & 1), which
    # a simple bank map predicts conflict-free, measures 2-way
    old = _linear_index(lambda r: (r & 7) ^ ((r >> 3) & 1))
    assert search[old] == 2
    assert sum(1 for d in search if d == 1) > 1000


def test_swizzle_permutes_chunks_of_each_row():
    for dtype in (0, 1, 2):
        rb = tkg.lds_row_bytes(dtype)
        seen = {}
        for p in bm.kernel_fragment_reads(dtype):
            for a in p:
                seen.setdefault(a // rb, set()).add(a % rb)
        for row, offs in seen.items():
            assert offs == set(range(0, rb, 16)), (dtype, row)


def test_fp4_scale_reads_measured_conflict_free():
    m = measured(bm.scale_read_pattern(8), 8)
    assert m is not None and m["degree"] == 1
