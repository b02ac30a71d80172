"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test below fixes part of the oracle with something independent of its
own code: closed forms of structured products (identity, permutation,
rank 1), exact rational arithmetic on tiny shapes, exact integer products,
format code tables and published special values, and planted mistakes that
the pins must catch.

The product definition (C = A x B, A: M x K, B: K x N, A row-major and B
column-major) is from page "ThunderKittens: Simple, Fast, and Adorable AI
Kernels", section 3.4 "Integration: How the Three Levels Compose into a
Complete Kernel", and page "ThunderKittens: 16x16 Tiles, ...", section
"Warp level: tiles are the only data structure".
"""
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from oracle.formats import (E2M1_TABLE, E4M3_TABLE, decode_bf16,
                            decode_e2m1_packed, decode_e4m3, round_to_bf16)


def _bf16_values(seed, r, c):
    return decode_bf16(gi.bf16_operand(seed, r, c))


# ------------------------------------------------------------------ GEMM

def test_identity_returns_operand():
    A = _bf16_values(1, 37, 53)
    C = oracle.gemm_f64(A, np.eye(53))
    assert np.array_equal(C, A)


def test_permutation_permutes_columns():
    # B = P with B[k, j] = 1 iff k == perm[j]  =>  C[:, j] = A[:, perm[j]]
    A = _bf16_values(2, 19, 40)
    perm = gi.permutation(3, 40)
    Bt = np.zeros((40, 40))
    Bt[np.arange(40), perm] = 1.0      # Bt[j, k] = B[k, j]
    C = oracle.gemm_f64(A, Bt)
    assert np.array_equal(C, A[:, perm])


def test_rank_one_closed_form():
    # A[i,k] = a_i u_k, B[k,j] = v_k b_j  =>  C[i,j] = a_i b_j (u . v),
    # exact for small integers.
    g = np.random.default_rng(4)
    a = g.integers(-5, 6, 23).astype(float)
    b = g.integers(-5, 6, 31).astype(float)
    u = g.integers(-4, 5, 64).astype(float)
    v = g.integers(-4, 5, 64).astype(float)
    A = np.outer(a, u)
    Bt = np.outer(b, v)
    C = oracle.gemm_f64(A, Bt)
    assert np.array_equal(C, np.outer(a, b) * float(u @ v))


def test_integer_products_exact():
    A = gi.small_integers(5, 33, 70)
    Bt = gi.small_integers(6, 17, 70)
    exact = A.astype(np.int64) @ Bt.astype(np.int64).T
    assert np.array_equal(oracle.gemm_f64(A, Bt), exact.astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (8, 7, 6),
                                   (15, 16, 17), (16, 33, 8), (3, 2, 33)])
def test_brute_force_against_exact_rationals(M, N, K):
    A = _bf16_values(10 + M, M, K)
    Bt = _bf16_values(20 + N, N, K)
    C = oracle.gemm_f64(A, Bt)
    u = 2.0 ** -53
    for i in range(M):
        for j in range(N):
            exact = sum((Fraction(A[i, k]) * Fraction(Bt[j, k])
                         for k in range(K)), Fraction(0))
            mag = sum(abs(A[i, k] * Bt[j, k]) for k in range(K))
            # recursive summation bound: |err| <= gamma_K * sum |a b|
            bound = K * u / (1 - K * u) * mag
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(bound)


def test_scale_applied_after_sum():
    A = _bf16_values(7, 9, 32)
    Bt = _bf16_values(8, 11, 32)
    base = oracle.gemm_f64(A, Bt)
    assert np.array_equal(oracle.gemm_f64(A, Bt, 0.25), base * 0.25)


def test_empty_and_degenerate_shapes():
    assert oracle.gemm_f64(np.zeros((0, 4)), np.zeros((3, 4))).shape == (0, 3)
    C = oracle.gemm_f64(np.zeros((2, 0)), np.zeros((3, 0)))
    assert C.shape == (2, 3) and not C.any()


def test_planted_transpose_is_caught():
    # A mistake planted in a copy of the oracle (B read row-major instead of
    # column-major) must fail the permutation pin.
    A = _bf16_values(2, 16, 16)
    perm = gi.permutation(3, 16)
    Bt = np.zeros((16, 16))
    Bt[np.arange(16), perm] = 1.0
    mutant = oracle.gemm_f64(A, np.ascontiguousarray(Bt.T))
    assert not np.array_equal(mutant, A[:, perm])


def test_planted_dropped_term_is_caught():
    # Dropping the last k of the sum must fail the integer pin.
    A = gi.small_integers(5, 8, 9)
    Bt = gi.small_integers(6, 8, 9)
    mutant = oracle.gemm_f64(A[:, :-1], Bt[:, :-1])
    exact = A.astype(np.int64) @ Bt.astype(np.int64).T
    assert not np.array_equal(mutant, exact)


# --------------------------------------------------------------- formats

def test_e4m3_special_values():
    # OCP e4m3: bias 7, 3 mantissa bits, max 448 at 0x7E, NaN at S.1111.111
    assert E4M3_TABLE[0x7E] == 448.0
    assert E4M3_TABLE[0x38] == 1.0
    assert E4M3_TABLE[0x08] == 2.0 ** -6           # smallest normal
    assert E4M3_TABLE[0x01] == 2.0 ** -9           # smallest subnormal
    assert E4M3_TABLE[0x07] == 7 * 2.0 ** -9       # largest subnormal
    assert np.isnan(E4M3_TABLE[0x7F]) and np.isnan(E4M3_TABLE[0xFF])
    assert E4M3_TABLE[0x00] == 0.0 and np.signbit(E4M3_TABLE[0x80])
    pos = E4M3_TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)                  # monotone codes
    assert np.array_equal(E4M3_TABLE[0x80:0xFF], -pos)


def test_e4m3_matches_torch_decode():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = decode_e4m3(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.array_equal(ref[~both_nan], mine[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))


def test_e2m1_table():
    # sign bit 3, exponent bits 2..1 with bias 1, one mantissa bit
    assert list(E2M1_TABLE[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(E2M1_TABLE[8:], -E2M1_TABLE[:8])


def test_e2m1_nibble_order():
    # element 2t in the low nibble of byte t
    packed = np.array([[0x72, 0x0F]], dtype=np.uint8)
    assert list(decode_e2m1_packed(packed)[0]) == [1.0, 6.0, -6.0, 0.0]


def test_bf16_decode_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    ref = ref.to(torch.float64).numpy()
    mine = decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.array_equal(np.isnan(ref), np.isnan(mine))


def test_round_to_bf16_ties_and_near_ties():
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing in [1, 2)
    cases = {
        one + ulp / 2: one,              # tie -> even (1.0)
        one + 3 * ulp / 2: one + 2 * ulp,  # tie -> even
        one + ulp / 2 + 2.0 ** -40: one + ulp,  # just above the tie
        one + ulp / 2 - 2.0 ** -40: one,
        -(one + ulp / 2): -one,
        2.0 ** -133: 2.0 ** -133,        # smallest subnormal
        1.5 * 2.0 ** -133: 2.0 ** -132,  # tie between 1 and 2 quanta -> 2
        2.0 ** -134: 0.0,                # tie between 0 and 1 quantum -> 0
        3.0e38 * 1.2: np.inf,            # past the largest finite bf16
    }
    for x, want in cases.items():
        got = round_to_bf16(np.array([x]))[0]
        assert got == want, (x, got, want)


def test_round_to_bf16_agrees_with_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x.astype(np.float64)), ref)


# ----------------------------------------------------- scaled formats

def test_fp4_blockscaled_dequant_uses_its_block_scale():
    # 32 elements per row = 2 blocks; block 0 scale 1.0 (0x38), block 1
    # scale 1.5 (0x3C). Code 0x7 is 6.0, code 0x1 is 0.5.
    codes = np.full((1, 32), 0x7, dtype=np.uint8)
    codes[0, 15] = 0x1
    codes[0, 16] = 0x1
    packed = gi.pack_nibbles(codes)
    scales = np.array([[0x38, 0x3C]], dtype=np.uint8)
    v = oracle.dequant_fp4_blockscaled(packed, scales)[0]
    assert v[0] == 6.0 and v[15] == 0.5
    assert v[16] == 0.75 and v[17] == 9.0 and v[31] == 9.0


def test_fp4_gemm_closed_form():
    # all values 1.0 (code 0x2) with block scale 2.0 (0x40) on A and 0.5
    # (0x30) on B, tensor scales 0.25 and 8: C = 2 * K * 1 * 0.25 * 8 ...
    M, N, K = 3, 5, 64
    A = gi.pack_nibbles(np.full((M, K), 0x2, np.uint8))
    B = gi.pack_nibbles(np.full((N, K), 0x2, np.uint8))
    As = np.full((M, K // 16), 0x40, np.uint8)
    Bs = np.full((N, K // 16), 0x30, np.uint8)
    C = oracle.gemm_fp4_blockscaled(A, As, 0.25, B, Bs, 8.0)
    assert np.all(C == K * (2.0 * 0.5) * 0.25 * 8.0)


def test_fp8_gemm_closed_form():
    M, N, K = 4, 6, 48
    A = np.full((M, K), 0x38, np.uint8)        # 1.0
    B = np.full((N, K), 0x40, np.uint8)        # 2.0
    C = oracle.gemm_fp8(A, 0.5, B, 3.0)
    assert np.all(C == K * 2.0 * 1.5)


def test_fp8_scale_is_product_of_fp32_scales():
    A = np.full((1, 16), 0x38, np.uint8)
    sa, sb = 0.1, 0.3                         # not exact in fp32
    C = oracle.gemm_fp8(A, sa, A, sb)
    want = 16 * float(np.float32(sa)) * float(np.float32(sb))
    assert C[0, 0] == want


# ------------------------------------------------------------- MX formats
# OCP Microscaling Formats v1.0 (external specification): E8M0 block
# scales 2^(e-127), blocks of 32 along K, e2m1 or e4m3 elements.

def test_e8m0_table():
    from oracle.formats import E8M0_TABLE, decode_e8m0
    import math
    for e in range(255):
        assert E8M0_TABLE[e] == math.ldexp(1.0, e - 127)
    assert np.isnan(E8M0_TABLE[255])
    assert decode_e8m0(np.array([127, 0, 254], np.uint8)).tolist() == [1.0, 2.0 ** -127, 2.0 ** 127]


def test_e8m0_matches_torch_decode():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e8m0fnu"):
        pytest.skip("torch has no float8_e8m0fnu")
    from oracle.formats import decode_e8m0
    codes = np.arange(255, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(decode_e8m0(codes), t)


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_mx_dequant_uses_its_block_scale(elem):
    # all elements 1.0, a different scale per block: the result shows each
    # element took the scale of block k // 32
    R, K = 3, 128
    one = 0x2 if elem == "e2m1" else 0x38
    codes = np.full((R, K), one, np.uint8)
    vals = gi.pack_nibbles(codes) if elem == "e2m1" else codes
    scales = (120 + np.arange(R * K // 32).reshape(R, K // 32)).astype(np.uint8)
    d = oracle.dequant_mx(vals, scales, elem)
    want = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    assert np.array_equal(d, want)


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_mx_gemm_against_exact_rationals(elem):
    g = np.random.default_rng(5)
    M, N, K = 3, 4, 64
    if elem == "e2m1":
        Ac, Bc = g.integers(0, 16, (M, K)).astype(np.uint8), g.integers(0, 16, (N, K)).astype(np.uint8)
        Av, Bv = gi.pack_nibbles(Ac), gi.pack_nibbles(Bc)
        ev = lambda c: Fraction(E2M1_TABLE[c])
    else:
        pool = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
        Ac, Bc = g.choice(pool, (M, K)), g.choice(pool, (N, K))
        Av, Bv = Ac, Bc
        ev = lambda c: Fraction(E4M3_TABLE[c])
    As = g.integers(110, 140, (M, K // 32)).astype(np.uint8)
    Bs = g.integers(110, 140, (N, K // 32)).astype(np.uint8)
    C = oracle.gemm_mx(Av, As, Bv, Bs, elem)
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    for i in range(M):
        for j in range(N):
            terms = [ev(Ac[i, k]) * Fraction(2) ** (int(As[i, k // 32]) - 127) *
                     ev(Bc[j, k]) * Fraction(2) ** (int(Bs[j, k // 32]) - 127)
                     for k in range(K)]
            exact = sum(terms)
            # recursive fp64 summation of exact products
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(gamma) * sum(abs(t) for t in terms)


def test_mx_planted_block_size_is_caught():
    # a dequantizer whose block boundaries sat 16 elements off (the 4-bit
    # format's block size) disagrees with the definition on a random case
    g = np.random.default_rng(8)
    codes = g.integers(0, 16, (2, 64)).astype(np.uint8)
    scales = g.integers(120, 135, (2, 2)).astype(np.uint8)
    good = oracle.dequant_mx(gi.pack_nibbles(codes), scales, "e2m1")
    from oracle.formats import decode_e2m1_packed as dec, decode_e8m0
    s16 = np.repeat(np.repeat(decode_e8m0(scales), 2, axis=1), 16, axis=1)[:, :64]
    planted = dec(gi.pack_nibbles(codes)) * np.roll(s16, 16, axis=1)
    assert not np.array_equal(good, planted)
    assert np.array_equal(good, dec(gi.pack_nibbles(codes)) * s16)


@pytest.mark.parametrize("elem", ["e2m1", "e4m3"])
def test_mx_quantize_round_trips_representable_values(elem):
    # values that are an element value times 2^e with one e per block come
    # back exactly
    g = np.random.default_rng(11)
    R, K = 4, 96
    table = E2M1_TABLE if elem == "e2m1" else E4M3_TABLE[np.isfinite(E4M3_TABLE)]
    base = g.choice(table, (R, K))
    base[:, ::32] = table.max()           # each block reaches the format maximum
    e = g.integers(-6, 7, (R, K // 32)).astype(np.float64)
    x = base * np.repeat(np.exp2(e), 32, axis=1)
    vals, scales = gi.mx_quantize(x, elem)
    assert np.array_equal(oracle.dequant_mx(vals, scales, elem), x)
