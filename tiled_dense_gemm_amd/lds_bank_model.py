"""CPU model of LDS bank conflicts for the pages' worked example, and the
fragment reads the gfx950 kernels issue.

Shared memory is split into banks of 4 bytes; the lanes of one phase of a
memory instruction that touch different 4-byte words of the same bank are
served one after another. The conflict degree of an instruction is the
largest number of distinct words any bank must serve in any phase (1 means
conflict-free).

* ``page_model`` is the H100 setting of page "ThunderKittens: 16x16 Tiles,
  ...", section "Warp level: tiles are the only data structure" (32 banks,
  phases of 8 threads for 16-byte accesses); it must reproduce the page's
  printed results, 8 for a row-major 128-byte-stride tile and 1 with the
  128-byte swizzle.
* gfx950 (MI355X) has no model here that predicts every measured degree.
  The kernels' layouts are chosen and checked by measurement: a probe
  kernel read every fragment pattern the kernels issue (as
  ``kernel_fragment_reads`` reports them from the library), and rocprofv3's
  SQ_LDS_BANK_CONFLICT per pattern gave the degrees recorded in
  tests/golden/lds_probe_gfx950.json. The functions below are the model
  classes those measurements were tested against: phases of 16 lanes for
  16-byte reads and 32 for 8- and 4-byte reads (measured), with banks from
  the 4-byte word index (``gfx950_word_bank``) or that index with address
  bits 9 and 10 folded into bank bit 2 (``gfx950_fold_bank``, the only
  linear fold of bits 8-10 that reproduces all 4096 measured 16x16
  row-swizzle reads). Each mispredicts some measured pattern (the tests
  show where), so the measured table is the check.
"""
from __future__ import annotations

from typing import Callable, List, Sequence

BANK_BYTES = 4


def conflict_degree(addrs: Sequence[int], access_bytes: int,
                    lanes_per_phase: int,
                    bank: Callable[[int], int]) -> int:
    """Worst number of distinct 4-byte words one bank serves in one phase.

    addrs: byte address of each lane (consecutive lanes form a phase);
    access_bytes: bytes each lane reads (multiple of 4, aligned);
    bank: byte address of a word -> bank index."""
    worst = 0
    for p0 in range(0, len(addrs), lanes_per_phase):
        words = {}
        for a in addrs[p0:p0 + lanes_per_phase]:
            for w in range(access_bytes // BANK_BYTES):
                word_addr = a + BANK_BYTES * w
                words.setdefault(bank(word_addr), set()).add(word_addr)
        worst = max(worst, max(len(s) for s in words.values()))
    return worst


def mod_bank(banks: int) -> Callable[[int], int]:
    return lambda a: (a // BANK_BYTES) % banks


# -- the page's H100 setting ------------------------------------------------

def page_swizzle(addr: int, span_bytes: int = 128) -> int:
    """The pages' byte swizzle: XOR the 16-byte chunk index with the
    128-byte row index inside a span of span_bytes * 8 bytes."""
    return addr ^ (((addr % (span_bytes * 8)) >> 7) << 4)


def page_model(row_stride: int, xform: Callable[[int], int] = lambda a: a) -> int:
    """32 threads each load 16 bytes of their own row; 32 banks; 4 phases of
    8 threads."""
    addrs = [xform(t * row_stride) for t in range(32)]
    return conflict_degree(addrs, 16, 8, mod_bank(32))


# -- the kernels' fragment reads ----------------------------------------------

def kernel_fragment_reads(dtype: int) -> List[List[int]]:
    """Every ds_read_b128 address pattern of the operand fragments the
    kernels issue for `dtype`, as reported by the library itself."""
    import tiled_dense_gemm_amd as tkg
    steps = tkg.lib.tkg_lds_fragment_offsets(
        dtype, 0, 0, 0, (tkg.ctypes.c_uint32 * 64)())
    if steps < 0:
        raise tkg.TkgError(steps, "tkg_lds_fragment_offsets")
    buf = (tkg.ctypes.c_uint32 * 64)()
    parts = 2 if tkg.lib.tkg_lds_fragment_offsets(dtype, 0, 1, 0, buf) > 0 else 1
    frags = 256 // tkg.lds_fragment_rows(dtype)
    return [tkg.lds_fragment_offsets(dtype, step, part, frag)
            for step in range(steps) for part in range(parts)
            for frag in range(frags)]


def scale_read_pattern(row_bytes: int = 8) -> List[int]:
    """LDS addresses of the 4-bit kernel's block-scale reads: lane l reads
    the 8 bytes of row l % 32 (rows `row_bytes` apart)."""
    return [(l % 32) * row_bytes for l in range(64)]



# -- gfx950: model classes the measurements rule out ----------------------------

GFX950_PHASE_LANES = {16: 16, 8: 32, 4: 32}   # measured: lanes per phase by access bytes


def gfx950_degree(addrs: Sequence[int], access_bytes: int,
                  bank: Callable[[int], int]) -> float:
    """Mean over the wave's phases of the most distinct words one bank
    serves (the measured degree: cycles over conflict-free cycles)."""
    ph = GFX950_PHASE_LANES[access_bytes]
    total = 0
    for p0 in range(0, len(addrs), ph):
        words = {}
        for a in addrs[p0:p0 + ph]:
            for w in range(access_bytes // BANK_BYTES):
                word_addr = a + BANK_BYTES * w
                words.setdefault(bank(word_addr), set()).add(word_addr)
        total += max(len(v) for v in words.values())
    return total / (len(addrs) // ph)


def gfx950_word_bank(a: int) -> int:
    """64 banks by 4-byte word index."""
    return (a // BANK_BYTES) % 64


def gfx950_fold_bank(a: int) -> int:
    """64 banks by word index, with address bits 9 and 10 XOR-ed into bank
    bit 2 (the 16-byte bank group's low bit)."""
    return gfx950_word_bank(a) ^ ((((a >> 9) ^ (a >> 10)) & 1) << 2)
