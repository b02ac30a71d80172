"""Number formats the oracle decodes -- TEST INFRASTRUCTURE, not the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything under ``oracle/``. The GPU path shares no
code with this module.

Every decoder maps the exact bytes the GPU receives to their exact real
value in IEEE double precision (all of these formats embed exactly in
fp64). The formats themselves are named, not specified, by the pages:

* bf16 -- the 16-bit brain-float operands of the tiled GEMM (page
  "ThunderKittens: Simple, Fast, and Adorable AI Kernels", section 3.4,
  "Warp-Level: Tile Operations": bf16 tiles accumulated in fp32). Layout: the
  upper half of an IEEE binary32.
* FP8 e4m3 -- page "ThunderKittens reaches 22.4 PFLOPS on NVIDIA Rubin"
  (opening paragraphs) and page 3 ("ThunderKittens DSL for GPU kernels",
  tile-abstraction section: the fp8 base tile is 16 x 32). Read as the OCP
  8-bit e4m3 ("fn") encoding: 1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, NaN only at S.1111.111, largest finite 448.
* e2m1 -- the 4-bit element of the block-scaled format (page "ThunderKittens
  reaches 22.4 PFLOPS on NVIDIA Rubin": NVFP4 is a block-scaled 4-bit float).
  1 sign bit (bit 3), 2 exponent bits with bias 1, 1 mantissa bit; no
  infinities or NaN; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.

* E8M0 -- the shared scale of an MX block (OCP Microscaling Formats
  specification v1.0, an external document; the pages' block-scaled idea,
  page "ThunderKittens reaches 22.4 PFLOPS on NVIDIA Rubin", "Feeding the
  faster tensor cores", in the form gfx950's scaled MFMA executes): an
  unsigned 8-bit exponent, value 2^(e - 127), 0xFF is NaN, no zero.

``round_to_bf16`` is the oracle's own round-to-nearest-even of an fp64 value
to bf16, used only to express the bf16 output rounding in comparisons.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact values (float64)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN payloads
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:  # subnormal: m/8 * 2^(1-7)
        return s * (m / 8.0) * 2.0 ** (-6)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _e2m1_value(code: int) -> float:
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:  # subnormal: m/2 * 2^(1-1)
        return s * (m / 2.0)
    return s * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def _e8m0_value(code: int) -> float:
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([_e8m0_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3 bytes (uint8) -> exact values (float64); 0x7F/0xFF -> NaN."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes (uint8) -> exact values 2^(e-127) (float64); 0xFF ->
    NaN."""
    return E8M0_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e2m1_packed(packed: np.ndarray) -> np.ndarray:
    """Packed e2m1 (uint8, R x K/2, element 2t in the low nibble of byte t)
    -> exact values (float64, R x K)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = E2M1_TABLE[p & 0xF]
    hi = E2M1_TABLE[p >> 4]
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even (one
    rounding, straight from fp64). Returns float64 holding bf16 values.
    bf16 has 8 significant bits, normal exponents down to -126 and
    subnormals with quantum 2^-133; magnitudes that round past the largest
    finite bf16 become infinities."""
    x = np.asarray(x, dtype=np.float64)
    mant, exp = np.frexp(x)            # x = mant * 2**exp, 0.5 <= |mant| < 1
    # quantum of the bf16 grid at this magnitude: 2^(exp-8) for normals,
    # never finer than the subnormal quantum 2^-133
    q_exp = np.maximum(exp - 8, -133)
    scaled = np.ldexp(x, -q_exp)       # exact: only shifts the exponent
    r = np.rint(scaled)                # round half to even
    out = np.ldexp(r, q_exp)
    big = np.abs(out) > 3.3895313892515355e38  # largest finite bf16
    out = np.where(big, np.copysign(np.inf, x), out)
    return np.where(x == 0, x, out)
