"""GPU parity at the largest K each product accepts.

A workgroup tile's rows of one operand are read through one buffer whose
size must stay below 2^31 bytes (256 rows x K x bytes per element), so the
C ABI caps K per format (include/tkg.h). These cases sit at that cap, where
per-lane row offsets pass 2^31 and every 32-bit offset computation is at
its limit. M = 256 fills one 256-row tile exactly; N = 200 leaves a ragged
tile (the bounds-checked instance).

At these K the oracle cannot finish even a sampled block in seconds, so the
operands have a closed-form product that holds at any size: A[i, k] = 1
where k = i (mod 5), B[j, k] = 1 where k = j (mod 7), 0 elsewhere, unit
scales. C[i, j] counts the k < K in the single residue class mod 35 that
both conditions select (5 and 7 are coprime): an integer below 2^24, so the
fp32 accumulation is exact and every output must equal the count rounded
to bf16, bit for bit. A row read at a wrong or wrapped offset, or zeros
read past a bound, changes counts.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import tiled_dense_gemm_amd as tkg
from oracle.formats import decode_bf16, round_to_bf16
from tests.parity import to_numpy_u16

pytestmark = pytest.mark.gpu

M, N = 256, 200
P_A, P_B = 5, 7
# the largest accepted K of each format (a multiple of its K granule)
K_BF16, K_FP8, K_FP4 = 4194296, 8388592, 16777152
K_MX = {"e2m1": 16777088, "e4m3": 8388480}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need the HIP device"
    return torch.device("cuda:0")


def _ones_where(rows, K, P, one, dev):
    """rows x K uint8/int16 codes: `one` where k = row (mod P), else 0."""
    k = torch.arange(K, device=dev, dtype=torch.int32) % P
    r = torch.arange(rows, device=dev, dtype=torch.int32) % P
    dtype = torch.int16 if one > 255 else torch.uint8
    out = torch.zeros((rows, K), dtype=dtype, device=dev)
    for r0 in range(0, rows, 32):
        out[r0:r0 + 32] = torch.where(k[None, :] == r[r0:r0 + 32, None],
                                      torch.tensor(one, dtype=dtype, device=dev),
                                      torch.tensor(0, dtype=dtype, device=dev))
    return out


def _packed_e2m1_ones(rows, K, P, dev):
    codes = _ones_where(rows, K, P, 0x2, dev)           # e2m1 0x2 = 1.0
    return codes[:, 0::2] | (codes[:, 1::2] << 4)       # element 2t in the low nibble


def _expected(K):
    """The counts, rounded to bf16 (float64 values)."""
    L = P_A * P_B
    crt = np.zeros((P_A, P_B), np.int64)
    for r in range(L):
        crt[r % P_A, r % P_B] = r
    r = crt[np.arange(M)[:, None] % P_A, np.arange(N)[None, :] % P_B]
    counts = np.where(r < K, (K - r + L - 1) // L, 0)
    assert counts.max() < 2 ** 24
    return round_to_bf16(counts.astype(np.float64))


def _check(C, K, what):
    G = decode_bf16(to_numpy_u16(C))
    E = _expected(K)
    bad = np.argwhere(G != E)
    assert bad.size == 0, (what, K, bad[:4].tolist(), G[tuple(bad[0])], E[tuple(bad[0])])


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_bf16_largest_k(dev):
    A = _ones_where(M, K_BF16, P_A, 0x3F80, dev).view(torch.bfloat16)
    B = _ones_where(N, K_BF16, P_B, 0x3F80, dev).view(torch.bfloat16)
    assert tkg.variant_info(tkg.DTYPE_BF16, 17)["tile"] == 256
    # automatic (128 x 128 tiles for this few) and a 256 x 256 configuration
    for v in (0, 17):
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        assert tkg.tkg_gemm_ex(tkg.DTYPE_BF16, M, N, K_BF16, A, None, 1.0, B, None, 1.0, C,
                               variant=v) == 0
        _check(C, K_BF16, ("bf16", v))
    del A, B
    _free()


def test_fp8_largest_k(dev):
    A = _ones_where(M, K_FP8, P_A, 0x38, dev)            # e4m3 0x38 = 1.0
    B = _ones_where(N, K_FP8, P_B, 0x38, dev)
    assert tkg.variant_info(tkg.DTYPE_FP8, 11)["tile"] == 256
    for v in (0, 11):
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        assert tkg.tkg_gemm_ex(tkg.DTYPE_FP8, M, N, K_FP8, A, None, 1.0, B, None, 1.0, C,
                               variant=v) == 0
        _check(C, K_FP8, ("fp8", v))
    del A, B
    _free()


def test_fp4_largest_k(dev):
    Ap = _packed_e2m1_ones(M, K_FP4, P_A, dev)
    Bp = _packed_e2m1_ones(N, K_FP4, P_B, dev)
    As = torch.full((M, K_FP4 // 16), 0x38, dtype=torch.uint8, device=dev)
    Bs = torch.full((N, K_FP4 // 16), 0x38, dtype=torch.uint8, device=dev)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    C = tkg.gemm_fp4_blockscaled(Ap, As, 1.0, Bp, Bs, 1.0, out=C)
    _check(C, K_FP4, "fp4")
    del Ap, Bp, As, Bs, C
    _free()


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_mx_largest_k(dev, elem):
    K = K_MX[elem]
    if elem == "e2m1":
        Av, Bv, gemm = _packed_e2m1_ones(M, K, P_A, dev), _packed_e2m1_ones(N, K, P_B, dev), \
            tkg.gemm_mxfp4
    else:
        Av, Bv, gemm = _ones_where(M, K, P_A, 0x38, dev), _ones_where(N, K, P_B, 0x38, dev), \
            tkg.gemm_mxfp8
    As = torch.full((M, K // 32), 127, dtype=torch.uint8, device=dev)   # E8M0 127 = 1.0
    Bs = torch.full((N, K // 32), 127, dtype=torch.uint8, device=dev)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    C = gemm(Av, As, Bv, Bs, out=C)
    _check(C, K, elem)
    del Av, Bv, As, Bs, C
    _free()
