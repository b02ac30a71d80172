"""LDS bank conflicts: the page's printed H100 model, and the MI355X
measurements that choose and check the kernels' swizzled layouts.

The gfx950 table (tests/golden/lds_probe_gfx950.json) was measured with a
probe kernel that issued each pattern and rocprofv3's SQ_LDS_BANK_CONFLICT
counter (profiles/lds_bank_probe_gfx950.md describes the run); every
fragment read the library reports must appear in it, address for address,
as conflict-free. The model classes tried against the table are tested
here too, each where it fails."""
import json
import os

import pytest

import tiled_dense_gemm_amd as tkg
from tiled_dense_gemm_amd import lds_bank_model as bm

GOLD = os.path.join(os.path.dirname(__file__), "golden")
PAGE = json.load(open(os.path.join(GOLD, "bank_model_page1.json")))
PROBE = json.load(open(os.path.join(GOLD, "lds_probe_gfx950.json")))
MEASURED = {(p["op"], p["bytes"], tuple(p["addresses"])): p for p in PROBE["patterns"]}


def measured(addrs, nbytes=16, op="r"):
    return MEASURED.get((op, nbytes, tuple(addrs)))


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
    un = [p for p in PROBE["patterns"] if " unswizzled " in p["name"]
          and not p["name"].startswith("4-bit values 16x16x32")]
    assert len(un) == 112
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


def test_fp4_16x16_reads_measured_conflicting():
    # the 16x16 fragment reads (row l % 16, chunk l / 16) measure 2-way on
    # the 64-byte-row swizzle; the 4-bit kernel keeps 32x32 blocks
    for kind in ("swizzled", "unswizzled"):
        pats = [p for p in PROBE["patterns"]
                if p["name"].startswith("4-bit values 16x16x32 %s " % kind)]
        assert len(pats) == 16 and all(p["degree"] == 2 for p in pats)


def test_mx_superstage_scale_reads_measured_conflict_free():
    # the MX kernels read each row's whole 16-byte superstage of scales
    # (rows 16 bytes apart, lane l row l % 32); reading one word or one
    # 8-byte pair of each row instead measures 4- and 2-way
    rows = [16 * (l % 32) for l in range(64)]
    assert measured(rows, 16)["degree"] == 1
    assert measured(rows, 4)["degree"] >= 4
    assert measured(rows, 8)["degree"] >= 2


FINISH_SHAPES = [(32, 4), (32, 2), (32, 1), (16, 8), (16, 4), (16, 2)]


@pytest.mark.parametrize("mi,rj", FINISH_SHAPES)
def test_finish_strip_measured_conflict_free(mi, rj):
    # every write and read of the finish's LDS strip, as the library
    # reports them, appears in the measured table without conflicts
    for kind, op in ((0, "w"), (1, "r")):
        n = tkg.lds_finish_count(mi, rj, kind)
        assert n > 0
        for i in range(n):
            m = measured(tkg.lds_finish_offsets(mi, rj, kind, i), 16, op)
            assert m is not None, (mi, rj, kind, i)
            assert m["degree"] == 1, m["name"]


def test_finish_rejected_layouts_measured_conflicting():
    for name in ("finish rejected padded rows b64 write", "finish rejected 128-byte rows xor write"):
        assert by_name(name)["degree"] >= 2


def _permlane_swap(x, y, width):
    # measured on gfx950 (v_permlane32_swap / v_permlane16_swap): the upper
    # `width` lanes of each 2*width group of x trade places with the lower
    # `width` lanes of the same group of y
    nx, ny = list(x), list(y)
    for g in range(0, 64, 2 * width):
        for i in range(width):
            nx[g + width + i], ny[g + i] = y[g + i], x[g + width + i]
    return nx, ny


@pytest.mark.parametrize("mi,rj", FINISH_SHAPES)
def test_finish_strip_moves_every_element_once(mi, rj):
    # Host model of the finish: accumulator block jj gives lane l row l % mi
    # and, in element group g, columns jj*mi + 4*(64/mi)*g + 4*(l // mi) ..
    # +3; lanes swap (32-wide for mi 32, 16-wide for mi 16) and write 16
    # bytes at the library's offsets; the reads at the library's offsets
    # must give lane l of read q the 8 columns rcol .. rcol+7 of row rrow.
    P, rb = 64 // mi, rj * mi * 2
    cpr, nr = rb // 16, mi * rb // 256
    lds = {}
    cols = lambda jj, g: [[(l % mi, jj * mi + 4 * P * g + 4 * (l // mi) + u) for u in range(4)]
                          for l in range(64)]
    if mi == 32:
        puts = [(cols(jj, 2 * p), cols(jj, 2 * p + 1)) for jj in range(rj) for p in range(2)]
    else:
        puts = [(cols(jj, 0), cols(jj + 1, 0)) for jj in range(0, rj, 2)]
    assert len(puts) == tkg.lds_finish_count(mi, rj, 0)
    for w, (X, Y) in enumerate(puts):
        lo = _permlane_swap([v[:2] for v in X], [v[:2] for v in Y], 32 if mi == 32 else 16)
        hi = _permlane_swap([v[2:] for v in X], [v[2:] for v in Y], 32 if mi == 32 else 16)
        offs = tkg.lds_finish_offsets(mi, rj, 0, w)
        for l in range(64):
            data = lo[0][l] + hi[0][l] + lo[1][l] + hi[1][l]
            assert 0 <= offs[l] and offs[l] + 16 <= mi * rb
            for k in range(8):
                assert offs[l] + 2 * k not in lds
                lds[offs[l] + 2 * k] = data[k]
    assert len(lds) == mi * rj * mi
    got = set()
    for q in range(tkg.lds_finish_count(mi, rj, 1)):
        offs = tkg.lds_finish_offsets(mi, rj, 1, q)
        for l in range(64):
            row = ((l % 16) // cpr) * nr + l // 16 + 4 * q
            col = 8 * ((l % 16) % cpr)
            for k in range(8):
                assert lds[offs[l] + 2 * k] == (row, col + k)
                got.add((row, col + k))
    assert len(got) == mi * rj * mi


def _search_addresses(A):
    # the measured 16x16 row-swizzle search: lane l reads row l % 16 of
    # 128-byte rows at chunk (l / 16) ^ mask(row), mask = A * bits(row)
    out = []
    for l in range(64):
        r = l % 16
        m = 0
        for b in range(3):
            m |= (bin(((A >> (4 * b)) & 15) & r).count("1") & 1) << b
        out.append(r * 128 + (((l // 16) ^ m) << 4))
    return out


def test_gfx950_word_index_model_ruled_out():
    # 64 banks by word index with the measured phase sizes predicts the
    # geometry patterns and the kernels' reads, but not the unswizzled
    # 16x16 reads of 128-byte rows: 8-way predicted, 4-way measured (the
    # hardware spreads rows 128 bytes apart over more banks)
    un = [p for p in PROBE["patterns"] if p["name"].startswith("bf16 16x16x32 unswizzled")]
    assert un and all(p["degree"] == 4 for p in un)
    assert all(bm.gfx950_degree(p["addresses"], 16, bm.gfx950_word_bank) == 8 for p in un)
    for p in PROBE["patterns"]:
        if p["op"] == "r" and (p["name"].startswith("b128 ") or " swizzled " in p["name"]) \
                and "16x16x32 swizzled" not in p["name"] and p["bytes"] == 16:
            assert bm.gfx950_degree(p["addresses"], 16, bm.gfx950_word_bank) == p["degree"], p["name"]


def test_gfx950_linear_fold_ruled_out():
    # Folding address bits 9 and 10 into bank bit 2 reproduces all 4096
    # measured 16x16 row-swizzle reads (of the 4096 linear folds of bits
    # 8..10 into the bank group, the only one that does) and the 4-way
    # unswizzled reads, but predicts the 16x16 reads of the 64-byte-row
    # layout conflict-free, which measure 2-way.
    search = PROBE["search_16x16_degrees"]
    for A in range(4096):
        assert bm.gfx950_degree(_search_addresses(A), 16, bm.gfx950_fold_bank) == search[A], A
    un = [p for p in PROBE["patterns"] if p["name"].startswith("bf16 16x16x32 unswizzled")]
    assert all(bm.gfx950_degree(p["addresses"], 16, bm.gfx950_fold_bank) == 4 for p in un)
    four_bit = by_name("4-bit values 16x16x32 swizzled step 0 part 0 frag 0")
    assert four_bit["degree"] == 2
    assert bm.gfx950_degree(four_bit["addresses"], 16, bm.gfx950_fold_bank) == 1
