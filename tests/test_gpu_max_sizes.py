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

Attention forward likewise at the most keys one head may hold (K and V
each just below 2^31 bytes), on a pattern whose softmax has a closed form
(below).
"""
import math

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


# ---------------------------------------------------------------- attention
# One head whose keys fill the largest K and V the entry point accepts (Nk
# rows of 2D bytes below 2^31): every query is e_0, K[j, 0] = +1 for even j
# and -1 for odd j (0 elsewhere), V[j, d] = ((j + d) mod 5) - 2, scale 1.
# The scores are +-1, so the softmax has a closed form built from residue
# counts of j mod 10 (tests/test_max_size_counts.py checks it against the
# oracle at small Nk). Nq = 40: two waves hold queries, two hold none.

NQ_ATTN = 40


def attention_closed_form(Nq, Nk, D):
    """(O, sum_j p_j |v_j|, lse) of the pattern above, fp64: O is Nq x D."""
    t = np.arange(10)
    cnt = np.where(t < Nk, (Nk - t + 9) // 10, 0).astype(np.float64)   # j = t mod 10
    w = np.where(t % 2 == 0, math.e, 1.0 / math.e)                      # exp(score)
    r = (t[:, None] + np.arange(D)[None, :]) % 5 - 2                     # v of class t
    Z = float(np.sum(cnt * w))
    num = (cnt * w) @ r
    mag = (cnt * w) @ np.abs(r)
    O = np.broadcast_to(num / Z, (Nq, D))
    A = np.broadcast_to(mag / Z, (Nq, D))
    return O, A, math.log(Z)


def _attn_pattern(Nq, Nk, D, dev):
    Q = torch.zeros((1, 1, Nq, D), dtype=torch.bfloat16, device=dev)
    Q[..., 0] = 1.0
    K = torch.zeros((1, 1, Nk, D), dtype=torch.bfloat16, device=dev)
    K[0, 0, 0::2, 0] = 1.0
    K[0, 0, 1::2, 0] = -1.0
    V = torch.empty((1, 1, Nk, D), dtype=torch.bfloat16, device=dev)
    d = torch.arange(D, device=dev, dtype=torch.int32)
    step = 1 << 20
    for j0 in range(0, Nk, step):
        j = torch.arange(j0, min(Nk, j0 + step), device=dev, dtype=torch.int32)
        V[0, 0, j0:j0 + j.numel()] = ((j[:, None] + d[None, :]) % 5 - 2).to(torch.bfloat16)
    return Q, K, V


@pytest.mark.parametrize("D", [128, 64])
def test_attention_largest_kv(dev, D):
    Nk = (2 ** 31 - 1) // (2 * D)          # the most keys one head may hold
    Q, K, V = _attn_pattern(NQ_ATTN, Nk, D, dev)
    O, lse = tkg.tkg_attention_fwd(Q, K, V, scale=1.0, lse=True)
    torch.cuda.synchronize()
    G = decode_bf16(to_numpy_u16(O))[0, 0]
    Glse = lse.cpu().numpy().astype(np.float64)[0, 0]
    R, A, Rlse = attention_closed_form(NQ_ATTN, Nk, D)
    bound = 2.0 ** -8 * (A + np.abs(R)) + 1e-6        # test_gpu_attention's tolerance
    assert np.all(np.abs(G - R) <= bound), (D, float(np.max(np.abs(G - R) - bound)))
    assert np.all(np.abs(Glse - Rlse) <= 2.0 ** -8 + 1e-6 * abs(Rlse)), (D, Glse[:2], Rlse)
    del Q, K, V, O, lse
    _free()


# The most queries one head may hold (Q and O each just below 2^31 bytes),
# over two key blocks: K[j, 0] = 1 (0 elsewhere), Q[i, 0] = (i mod 3) - 1,
# so every score of row i is ((i mod 3) - 1) * scale, the softmax of every
# row is uniform and O[i] is the mean of V's rows, while lse[i] =
# ((i mod 3) - 1) * scale + ln Nk checks each row's own Q. O starts as NaN.

NK_WIDE = 64


def uniform_rows_closed_form(Nk, D, scale, rows):
    """(O row, lse of the given row indices) of the pattern above, fp64."""
    j, d = np.arange(Nk)[:, None], np.arange(D)[None, :]
    O = ((j + d) % 5 - 2).mean(axis=0)
    lse = ((np.asarray(rows) % 3) - 1) * scale + math.log(Nk)
    return O, lse


@pytest.mark.parametrize("D", [128, 64])
def test_attention_largest_q(dev, D):
    Nq = (2 ** 31 - 1) // (2 * D)          # the most queries one head may hold
    scale = 1.0 / math.sqrt(D)
    Q = torch.zeros((1, 1, Nq, D), dtype=torch.bfloat16, device=dev)
    Q[0, 0, :, 0] = ((torch.arange(Nq, device=dev) % 3) - 1).to(torch.bfloat16)
    K = torch.zeros((1, 1, NK_WIDE, D), dtype=torch.bfloat16, device=dev)
    K[..., 0] = 1.0
    j = torch.arange(NK_WIDE, device=dev)[:, None]
    d = torch.arange(D, device=dev)[None, :]
    V = ((j + d) % 5 - 2).to(torch.bfloat16)[None, None]
    O = torch.full((1, 1, Nq, D), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((1, 1, Nq), float("nan"), dtype=torch.float32, device=dev)
    tkg.tkg_attention_fwd(Q, K, V, scale=scale, out=O, lse=lse)
    torch.cuda.synchronize()
    Oref, _ = uniform_rows_closed_form(NK_WIDE, D, scale, [0])
    # every row equals the mean of V's rows within one bf16 rounding
    Of = O[0, 0].float()
    assert bool(torch.isfinite(Of).all()), D
    ref = torch.tensor(Oref, dtype=torch.float32, device=dev)
    err = (Of - ref[None, :]).abs().max().item()
    assert err <= 2.0 ** -8 * float(np.abs(Oref).max()) + 1e-6, (D, err)
    # lse of every row: its own Q entry sets the score
    rows = torch.arange(Nq, device=dev)
    lref = ((rows % 3) - 1).double() * scale + math.log(NK_WIDE)
    lerr = (lse[0, 0].double() - lref).abs().max().item()
    assert lerr <= 2.0 ** -8 + 1e-6 * (abs(scale) + math.log(NK_WIDE)), (D, lerr)
    del Q, K, V, O, lse, Of, rows, lref
    _free()
