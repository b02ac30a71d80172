"""Seeded synthetic operands for the tiled dense GEMM and attention forward.

This module is shared by the GPU path's tests and benchmark and by the
oracle's tests. It holds none of the product's arithmetic: it only draws
numbers and encodes them into the operand formats the library consumes.
Decoding those bytes back into values is done independently on each side
(the GPU kernels in hardware, the oracle from the format definitions).

Workloads (synthetic operand shapes, as the pages' GEMM benchmarks use):
entries i.i.d. N(0, 1) (optionally divided by sqrt(K)); fp8 operands are
quantized with one fp32 scale per tensor, s = amax/448; the block-scaled
4-bit operands follow ``fp4_operand``'s recipe. A uses ``seed`` and B uses
``seed + 1`` by convention of the callers.

Attention operands (``attention_operands``): Q [B, Hq, Nq, D] and K, V
[B, Hkv, Nk, D] with i.i.d. N(0, std^2) entries rounded to bf16, Q from
``seed``, K from ``seed + 1``, V from ``seed + 2``.

Layouts: A is M x K row-major; B is handed over column-major, i.e. as an
N x K row-major array ("Bt"). Both are K-contiguous.

Random numbers come from numpy's Philox (a counter-based generator), so the
same seed gives the same operand on every machine. ``device`` builds the
same kinds of operands on the GPU with torch's generator for sizes the host
cannot draw quickly; those are seeded too but are not bit-identical to the
host ones.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
FP4_BLOCK = 16
MX_BLOCK = 32
# largest power of two that the element formats' maxima reach: 6 = 1.5 * 2^2
# (e2m1), 448 = 1.75 * 2^8 (e4m3)
MX_EMAX = {"e2m1": 2, "e4m3": 8}


def normal(seed: int, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """rows x cols i.i.d. N(0, std^2) draws in float64 (Philox, key = seed)."""
    g = np.random.Generator(np.random.Philox(key=int(seed)))
    x = g.standard_normal((rows, cols), dtype=np.float64)
    if std != 1.0:
        x *= std
    return x


# ----------------------------------------------------------------- encoders

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), round to nearest even via
    binary32 (an input-side encoding: double rounding in rare ties only
    changes which bf16 value is drawn, not parity)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def _pos_e4m3_values() -> np.ndarray:
    # the 127 non-negative finite codes 0x00..0x7E, in increasing order
    codes = np.arange(0x7F)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6,
                    (1.0 + m / 8.0) * np.exp2(e - 7.0))


_E4M3_POS = _pos_e4m3_values()


def e4m3_codes(y: np.ndarray) -> np.ndarray:
    """float64 -> OCP e4m3 codes (uint8): round to nearest even, saturate to
    +-448 (never NaN for finite input)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    _, ex = np.frexp(a)                   # a = f * 2^ex, 0.5 <= f < 1
    q = np.maximum(ex - 4, -9)            # grid spacing 2^(E-3), E = ex-1
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.minimum(r, E4M3_MAX)
    code = np.searchsorted(_E4M3_POS, r).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 7)


_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_codes(y: np.ndarray) -> np.ndarray:
    """float64 -> e2m1 nibbles (uint8 in 0..15): round to nearest even,
    saturate to +-6."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E2M1_MAX)
    _, ex = np.frexp(a)
    q = np.maximum(ex - 2, -1)            # spacing 2^(E-1), at least 0.5
    r = np.ldexp(np.rint(np.ldexp(a, -q)), q)
    r = np.minimum(r, E2M1_MAX)
    code = np.searchsorted(_E2M1_POS, r).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 3)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """R x K nibbles -> R x K/2 bytes, element 2t in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


# ---------------------------------------------------------------- operands

def bf16_operand(seed: int, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    """Seeded bf16 operand (uint16 bits, rows x cols)."""
    return bf16_bits(normal(seed, rows, cols, std))


def fp8_quantize(x: np.ndarray):
    """Per-tensor e4m3 quantization: s = fp32(amax/448), codes of x/s.
    Returns (uint8 codes, float scale)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    return e4m3_codes(x / np.float64(s)), float(s)


def fp8_operand(seed: int, rows: int, cols: int, std: float = 1.0):
    """Seeded fp8 operand: (uint8 e4m3 codes rows x cols, fp32 scale)."""
    return fp8_quantize(normal(seed, rows, cols, std))


def fp4_quantize(x: np.ndarray, block: int = FP4_BLOCK):
    """Block-scaled 4-bit quantization along the last axis (K):
    t = fp32(amax / (6 * 448)); each block of ``block`` elements gets the
    e4m3 scale sb = e4m3(amax_block / (6 t)); elements become
    e2m1(x / (sb * t)) (0 where sb is 0).
    Returns (packed uint8 R x K/2, scales uint8 R x K/block, float t)."""
    R, K = x.shape
    if K % block or K % 2:
        raise ValueError("K=%d must be a multiple of %d" % (K, block))
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    t = np.float32(amax / (E2M1_MAX * E4M3_MAX)) if amax > 0 else np.float32(1.0)
    xb = x.reshape(R, K // block, block)
    bmax = np.max(np.abs(xb), axis=2)
    sc = e4m3_codes(bmax / (E2M1_MAX * np.float64(t)))
    sval = np.where(sc & 0x78 == 0, (sc & 7) / 8.0 * 2.0 ** -6,
                    (1.0 + (sc & 7) / 8.0) * np.exp2(((sc >> 3) & 0xF) - 7.0))
    denom = sval[..., None] * np.float64(t)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(denom > 0, xb / np.where(denom > 0, denom, 1.0), 0.0)
    codes = e2m1_codes(y.reshape(R, K))
    return pack_nibbles(codes), sc, float(t)


def fp4_operand(seed: int, rows: int, cols: int, std: float = 1.0):
    """Seeded block-scaled 4-bit operand: (packed, scales, tensor scale)."""
    return fp4_quantize(normal(seed, rows, cols, std))


def mx_quantize(x: np.ndarray, elem: str):
    """MX quantization along the last axis (K), in the OCP MX recipe: each
    block of 32 gets the shared exponent e = floor(log2(amax_block)) -
    emax(elem), stored as the E8M0 byte e + 127 (clamped to 0..254; a zero
    block gets 0), and its elements become elem(x / 2^e), rounded to
    nearest even and saturated.
    Returns (values: R x K/2 packed e2m1 or R x K e4m3 codes, scales R x K/32)."""
    R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K=%d must be a multiple of %d" % (K, MX_BLOCK))
    xb = x.reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(xb), axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), -127.0)
    e = np.clip(e - MX_EMAX[elem] * (amax > 0), -127, 127).astype(np.int64)
    scales = (e + 127).astype(np.uint8)
    y = (xb / np.exp2(e.astype(np.float64))[..., None]).reshape(R, K)
    if elem == "e2m1":
        return pack_nibbles(e2m1_codes(y)), scales
    return e4m3_codes(y), scales


def mx_operand(seed: int, rows: int, cols: int, elem: str, std: float = 1.0):
    """Seeded MX operand: (values, E8M0 scales)."""
    return mx_quantize(normal(seed, rows, cols, std), elem)


def attention_operands(seed: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int,
                       D: int, std_q: float = 1.0, std_kv: float = 1.0):
    """Seeded bf16 attention inputs (uint16 bits): Q [B, Hq, Nq, D],
    K and V [B, Hkv, Nk, D]."""
    q = bf16_operand(seed, B * Hq * Nq, D, std_q).reshape(B, Hq, Nq, D)
    k = bf16_operand(seed + 1, B * Hkv * Nk, D, std_kv).reshape(B, Hkv, Nk, D)
    v = bf16_operand(seed + 2, B * Hkv * Nk, D, std_kv).reshape(B, Hkv, Nk, D)
    return q, k, v


# ----------------------------------------------------- structured operands

def identity_bits_bf16(n: int) -> np.ndarray:
    """n x n identity as bf16 bits (1.0 = 0x3F80)."""
    out = np.zeros((n, n), dtype=np.uint16)
    np.fill_diagonal(out, 0x3F80)
    return out


def permutation(seed: int, n: int) -> np.ndarray:
    """A seeded permutation of 0..n-1."""
    g = np.random.Generator(np.random.Philox(key=int(seed)))
    return g.permutation(n)


def small_integers(seed: int, rows: int, cols: int, lo: int = -8,
                   hi: int = 8) -> np.ndarray:
    """rows x cols integers drawn uniformly from [lo, hi], as float64."""
    g = np.random.Generator(np.random.Philox(key=int(seed)))
    return g.integers(lo, hi + 1, size=(rows, cols)).astype(np.float64)
