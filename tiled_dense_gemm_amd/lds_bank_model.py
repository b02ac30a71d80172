"""CPU model of LDS bank conflicts, used to prove the kernels' swizzled
layouts conflict-free.

Shared memory is split into banks of 4 bytes; the lanes of one phase of a
memory instruction that touch different 4-byte words of the same bank are
served one after another. The conflict degree of an instruction is the
largest number of distinct words any bank must serve in any phase (1 means
conflict-free). Page "ThunderKittens: 16x16 Tiles, ...", section "Warp
level: tiles are the only data structure", models H100 this way (32 banks,
phases of 8 threads for 16-byte accesses) and reports 8 for a row-major
128-byte-stride tile and 1 with the 128-byte swizzle; ``page_model`` below is
that setting, kept as a test fixture.

For gfx950 two geometries are considered, because the phase grouping of
``ds_read_b128`` is not documented: 32 banks with phases of 8 lanes (as on
earlier CDNA parts) and 64 banks with phases of 16 lanes (doubled LDS
bandwidth). The kernels' layouts are checked to be conflict-free in both;
the SQ_LDS_BANK_CONFLICT counter measures the real chip.
"""
from __future__ import annotations

from typing import Callable, Iterable, List, Sequence

BANK_BYTES = 4

# (banks, lanes per phase for a 16-byte access)
GFX950_GEOMETRIES = {"32 banks x 8 lanes": (32, 8), "64 banks x 16 lanes": (64, 16)}


def conflict_degree(addrs: Sequence[int], access_bytes: int, banks: int,
                    lanes_per_phase: int) -> int:
    """Worst number of distinct words one bank serves in one phase.

    addrs: byte address of each lane (consecutive lanes form a phase);
    access_bytes: bytes each lane reads (multiple of 4, aligned)."""
    worst = 0
    for p0 in range(0, len(addrs), lanes_per_phase):
        words_per_bank = {}
        for a in addrs[p0:p0 + lanes_per_phase]:
            for w in range(access_bytes // BANK_BYTES):
                word = a // BANK_BYTES + w
                words_per_bank.setdefault(word % banks, set()).add(word)
        worst = max(worst, max(len(s) for s in words_per_bank.values()))
    return worst


def phase_lanes(access_bytes: int, banks: int) -> int:
    """Lanes per phase: one phase moves one word per bank."""
    return banks * BANK_BYTES // access_bytes


# -- the page's H100 setting ----------------------------------------------

def page_swizzle(addr: int, span_bytes: int = 128) -> int:
    """The pages' byte swizzle: XOR the 16-byte chunk index with the
    128-byte row index inside a span of span_bytes * 8 bytes."""
    return addr ^ (((addr % (span_bytes * 8)) >> 7) << 4)


def page_model(row_stride: int, xform: Callable[[int], int] = lambda a: a) -> int:
    """32 threads each load 16 bytes of their own row; 32 banks; 4 phases of
    8 threads."""
    addrs = [xform(t * row_stride) for t in range(32)]
    return conflict_degree(addrs, 16, 32, 8)


# -- the kernels' fragment reads ----------------------------------------------

def kernel_fragment_reads(dtype: int) -> List[List[int]]:
    """Every ds_read_b128 address pattern of the operand fragments the
    kernels issue for `dtype`, as reported by the library itself."""
    import tiled_dense_gemm_amd as tkg
    steps = tkg.lib.tkg_lds_fragment_offsets(
        dtype, 0, 0, 0, (tkg.ctypes.c_uint32 * 64)())
    if steps < 0:
        raise tkg.TkgError(steps, "tkg_lds_fragment_offsets")
    parts = 2 if dtype == tkg.DTYPE_FP8 else 1
    return [tkg.lds_fragment_offsets(dtype, step, part, frag)
            for step in range(steps) for part in range(parts)
            for frag in range(8)]


def worst_degree(patterns: Iterable[Sequence[int]], access_bytes: int,
                 banks: int, lanes: int) -> int:
    return max(conflict_degree(p, access_bytes, banks, lanes) for p in patterns)


def scale_read_pattern(row_bytes: int = 8, read_bytes: int = 8) -> List[int]:
    """LDS addresses of the 4-bit kernel's block-scale reads: lane l reads
    `read_bytes` of row l % 32 (rows `row_bytes` apart)."""
    return [(l % 32) * row_bytes for l in range(64)]
