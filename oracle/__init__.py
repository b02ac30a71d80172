"""CPU oracle for the tiled dense GEMM -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call, link or execute anything under ``oracle/``.
The product path never does, and the oracle shares no code with the GPU
library (no kernels, headers, helpers or tables); both sides only consume
the same seeded inputs from ``gemm_inputs``.

What it computes is the plain definition of the product on the exact values
of the bytes the GPU receives, accumulated in IEEE fp64:

    C[i, j] = s * sum_k  A[i, k] * B[k, j]

* C = A x B with A of size M x K, B of size K x N and C of size M x N: page
  "ThunderKittens: Simple, Fast, and Adorable AI Kernels", section 3.4,
  "Integration: How the Three Levels Compose into a Complete Kernel"
  (grid-level paragraph).
* A row-major, B column-major (the operand layouts of mma_AB): page
  "ThunderKittens: 16x16 Tiles, the Load-Compute-Store-Finish Template, and
  Why 40 Lines Can Match cuBLAS", section "Warp level: tiles are the only
  data structure". B is therefore handed over as an N x K array ``Bt``.
* bf16 operands with fp32 accumulation: same page 2 section 3.4,
  "Warp-Level: Tile Operations". The oracle accumulates in fp64 instead,
  which is the exact-up-to-rounding target the fp32 path approximates.
* FP8 and the block-scaled 4-bit format: page "ThunderKittens reaches 22.4
  PFLOPS on NVIDIA Rubin", opening paragraphs and "Feeding the faster tensor
  cores" (block-scaling factors travel with the 4-bit values).
  Readings where the pages are silent: fp8 carries one fp32 scale per tensor
  and the result is multiplied by s = sA * sB after the sum; the 4-bit
  format is e2m1 values in blocks of 16 along K, each block with an e4m3
  scale, plus one fp32 scale per tensor, s = tA * tB.

* MX block-scaled operands (the gfx950-native form of block scaling; OCP
  Microscaling Formats v1.0, an external specification): elements e2m1
  ("MXFP4", two per byte, element 2t in the low nibble of byte t) or OCP
  e4m3 ("MXFP8"), in blocks of 32 along K, each block with one E8M0 scale
  2^(e-127); value[r, k] = element[r, k] * scale[r, k // 32], no per-tensor
  scale.

Pins (see tests/test_oracle_pins.py): identity, permutation and rank-1
closed forms, brute force against exact rational arithmetic on tiny shapes,
integer-exact products, and code tables of every decoder.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .formats import (decode_bf16, decode_e2m1_packed, decode_e4m3,
                      decode_e8m0, round_to_bf16, E2M1_TABLE, E4M3_TABLE,
                      E8M0_TABLE)

__all__ = [
    "gemm_f64", "gemm_bf16", "gemm_fp8", "gemm_fp4_blockscaled",
    "dequant_fp4_blockscaled", "dequant_mx", "gemm_mx", "MX_BLOCK",
    "abs_gemm_f64", "decode_bf16", "decode_e4m3", "decode_e8m0",
    "decode_e2m1_packed", "round_to_bf16", "num_threads",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def _load():
    global _lib
    if _lib is None:
        from . import _build
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.ref_gemm_f64.restype = None
        lib.ref_gemm_f64.argtypes = [
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p]
        lib.ref_gemm_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the reference GEMM's parallel loop uses."""
    return int(_load().ref_gemm_num_threads())


def gemm_f64(A: np.ndarray, Bt: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """C = scale * A @ Bt.T in fp64, k summed in order (C library).

    A: M x K, Bt: N x K (B in column-major order); any real dtype, converted
    to float64 exactly."""
    A = np.ascontiguousarray(A, dtype=np.float64)
    Bt = np.ascontiguousarray(Bt, dtype=np.float64)
    M, K = A.shape
    N, K2 = Bt.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    C = np.empty((M, N), dtype=np.float64)
    if M and N:
        _load().ref_gemm_f64(M, N, K, A.ctypes.data, Bt.ctypes.data,
                             float(scale), C.ctypes.data)
    return C


def abs_gemm_f64(A: np.ndarray, Bt: np.ndarray) -> np.ndarray:
    """(|A| |B|)[i, j] = sum_k |A[i, k]| |B[k, j]|, the magnitude that sets the
    per-element error bound of a reduced-precision product."""
    return gemm_f64(np.abs(np.asarray(A, dtype=np.float64)),
                    np.abs(np.asarray(Bt, dtype=np.float64)))


def gemm_bf16(A_bits: np.ndarray, Bt_bits: np.ndarray) -> np.ndarray:
    """bf16 operands (uint16 bit patterns, A: M x K, Bt: N x K) -> exact-input
    fp64 product, not rounded to the bf16 output."""
    return gemm_f64(decode_bf16(A_bits), decode_bf16(Bt_bits))


def gemm_fp8(A_codes: np.ndarray, scale_a: float, Bt_codes: np.ndarray,
             scale_b: float) -> np.ndarray:
    """OCP e4m3 operands (uint8, A: M x K, Bt: N x K) with one fp32 scale per
    tensor -> sA * sB * (A @ B) in fp64."""
    s = float(np.float32(scale_a)) * float(np.float32(scale_b))  # exact in fp64
    return gemm_f64(decode_e4m3(A_codes), decode_e4m3(Bt_codes), s)


def dequant_fp4_blockscaled(packed: np.ndarray, scales: np.ndarray,
                            block: int = 16) -> np.ndarray:
    """Block-scaled 4-bit operand -> exact fp64 values without the per-tensor
    scale: value[r, k] = e2m1(packed)[r, k] * e4m3(scales[r, k // block]).

    packed: R x K/2 uint8 (element 2t in the low nibble of byte t);
    scales: R x K/block uint8 (e4m3)."""
    v = decode_e2m1_packed(packed)
    s = decode_e4m3(scales)
    R, K = v.shape
    if s.shape != (R, K // block) or K % block:
        raise ValueError("scale shape %r does not match %d x %d/%d"
                         % (s.shape, R, K, block))
    return v * np.repeat(s, block, axis=1)


def gemm_fp4_blockscaled(A_packed, A_scales, tensor_scale_a, B_packed,
                         B_scales, tensor_scale_b) -> np.ndarray:
    """Block-scaled 4-bit operands (A: M x K, Bt: N x K, see
    ``dequant_fp4_blockscaled``) with one fp32 scale per tensor ->
    tA * tB * (A @ B) in fp64."""
    s = float(np.float32(tensor_scale_a)) * float(np.float32(tensor_scale_b))
    return gemm_f64(dequant_fp4_blockscaled(A_packed, A_scales),
                    dequant_fp4_blockscaled(B_packed, B_scales), s)


MX_BLOCK = 32


def dequant_mx(values: np.ndarray, scales: np.ndarray, elem: str) -> np.ndarray:
    """MX operand -> exact fp64 values: element(values)[r, k] *
    e8m0(scales)[r, k // 32].

    values: R x K/2 uint8 packed e2m1 (elem "e2m1") or R x K uint8 OCP e4m3
    (elem "e4m3"); scales: R x K/32 uint8 E8M0."""
    if elem == "e2m1":
        v = decode_e2m1_packed(values)
    elif elem == "e4m3":
        v = decode_e4m3(values)
    else:
        raise ValueError("element format %r" % (elem,))
    s = decode_e8m0(scales)
    R, K = v.shape
    if K % MX_BLOCK or s.shape != (R, K // MX_BLOCK):
        raise ValueError("scale shape %r does not match %d x %d/%d"
                         % (s.shape, R, K, MX_BLOCK))
    return v * np.repeat(s, MX_BLOCK, axis=1)


def gemm_mx(A_values, A_scales, B_values, B_scales, elem: str) -> np.ndarray:
    """MX operands (A: M x K, Bt: N x K, see ``dequant_mx``) -> A @ B in
    fp64."""
    return gemm_f64(dequant_mx(A_values, A_scales, elem),
                    dequant_mx(B_values, B_scales, elem))
