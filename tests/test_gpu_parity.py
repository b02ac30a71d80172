"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Tolerances:
* bf16: relative Frobenius error <= 1e-3 against the oracle rounded to bf16
  (rounding the exact product to bf16 alone costs ~1.7e-3 against the
  unrounded one, so the bound applies to the rounded reference), and per
  element |G - C| <= 1e-2 * (|A||B|)_ij + 1e-3 against the unrounded oracle.
* fp8 and block-scaled 4-bit: relative Frobenius error <= 2e-2 against the
  oracle on the same dequantized inputs.
* Integer-valued and structured inputs (identity, permutation, small
  integers) make fp32 accumulation exact, so there the result must equal the
  oracle rounded to bf16 bit for bit.
Large shapes are checked on 64x64 output tiles (corners, tiles straddling
workgroup-tile boundaries, random ones), each tile on its own.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gemm_inputs as gi
import gemm_inputs.device  # noqa: F401  (gi.device)
import oracle
import tiled_dense_gemm_amd as tkg
from oracle.formats import decode_bf16, decode_e4m3, round_to_bf16
from tests.parity import relfro, sample_tiles, to_numpy_u16, to_numpy_u8

pytestmark = pytest.mark.gpu

BF16_RELFRO = 1e-3
BF16_ELEM_REL, BF16_ELEM_ABS = 1e-2, 1e-3
LOWP_RELFRO = 2e-2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need the HIP device"
    return torch.device("cuda:0")


def _up(a, dev, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t if dtype is None else t.view(dtype)


def _bf16_result(C):
    return decode_bf16(to_numpy_u16(C))


def check_bf16(G, A64, Bt64, what=""):
    R = oracle.gemm_f64(A64, Bt64)
    err = relfro(G, round_to_bf16(R))
    assert err <= BF16_RELFRO, (what, err)
    bound = BF16_ELEM_REL * oracle.abs_gemm_f64(A64, Bt64) + BF16_ELEM_ABS
    assert np.all(np.abs(G - R) <= bound), (what, float(np.max(np.abs(G - R) - bound)))
    return err


def lowp_elem_bound(absprod, K):
    """Per-element bound for products of exactly representable operands
    (fp8 and 4-bit): each product is exact in fp32, the fp32 sum of K terms
    is off by at most K 2^-24 (|A||B|)_ij, the fp32 scale multiply by 2^-24
    relative, and the bf16 rounding by 2^-9 relative:
    |G - C| <= (2^-9 + (K + 2) 2^-24) (|A||B|)_ij (x 1.001 for the bound's
    own rounding)."""
    return (2.0 ** -9 + (K + 2) * 2.0 ** -24) * 1.001 * absprod + 1e-30


def check_fp8_elementwise(G, a, sa, b, sb, what=""):
    """fp8: relative Frobenius <= 2e-2 against the oracle on the same
    dequantized inputs (the stated tolerance) and the per-element bound of
    lowp_elem_bound."""
    R = oracle.gemm_fp8(a, sa, b, sb)
    err = relfro(G, R)
    assert err <= LOWP_RELFRO, (what, err)
    Ad = decode_e4m3(a) * float(sa)
    Bd = decode_e4m3(b) * float(sb)
    bound = lowp_elem_bound(oracle.abs_gemm_f64(Ad, Bd), a.shape[1])
    assert np.all(np.abs(G - R) <= bound), (what, float(np.max(np.abs(G - R) - bound)))
    return err


# ----------------------------------------------------------------- bf16

def test_bf16_identity_bit_exact(dev):
    M, K = 300, 512
    A = gi.bf16_operand(1, M, K)
    C = tkg.gemm_bf16(_up(A, dev, torch.bfloat16),
                      _up(gi.identity_bits_bf16(K), dev, torch.bfloat16))
    assert np.array_equal(to_numpy_u16(C), A)


def test_bf16_permutation_bit_exact(dev):
    M, K = 256, 768
    A = gi.bf16_operand(2, M, K)
    perm = gi.permutation(3, K)
    Bt = np.zeros((K, K), np.uint16)
    Bt[np.arange(K), perm] = 0x3F80              # B[perm[j], j] = 1
    C = tkg.gemm_bf16(_up(A, dev, torch.bfloat16), _up(Bt, dev, torch.bfloat16))
    assert np.array_equal(to_numpy_u16(C), A[:, perm])


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (300, 260, 136),
                                   (1, 1, 8), (257, 255, 1032)])
def test_bf16_integers_bit_exact(dev, M, N, K):
    A = gi.small_integers(4, M, K)
    Bt = gi.small_integers(5, N, K)
    C = tkg.gemm_bf16(_up(gi.bf16_bits(A), dev, torch.bfloat16),
                      _up(gi.bf16_bits(Bt), dev, torch.bfloat16))
    assert np.array_equal(_bf16_result(C), round_to_bf16(oracle.gemm_f64(A, Bt)))


def test_bf16_rank_one_bit_exact(dev):
    # A[i,k] = a_i u_k, B[k,j] = v_k b_j with powers of two: C is exact
    M, N, K = 320, 288, 256
    g = np.random.default_rng(7)
    a = 2.0 ** g.integers(-3, 4, M); u = 2.0 ** g.integers(-3, 4, K)
    b = 2.0 ** g.integers(-3, 4, N); v = g.choice([-1.0, 1.0], K)
    A, Bt = np.outer(a, u), np.outer(b, v)
    C = tkg.gemm_bf16(_up(gi.bf16_bits(A), dev, torch.bfloat16),
                      _up(gi.bf16_bits(Bt), dev, torch.bfloat16))
    assert np.array_equal(_bf16_result(C), round_to_bf16(np.outer(a, b) * float(u @ v)))


def test_bf16_normal_256(dev):
    # the small configuration: 256^3, entries N(0, 1)
    A = gi.bf16_operand(0, 256, 256)
    Bt = gi.bf16_operand(1, 256, 256)
    C = tkg.gemm_bf16(_up(A, dev, torch.bfloat16), _up(Bt, dev, torch.bfloat16))
    G = _bf16_result(C)
    check_bf16(G, decode_bf16(A), decode_bf16(Bt), "256^3")
    # statistical pin: against the unrounded product the error is the bf16
    # output rounding, ~1.7e-3; much more would mean accumulation damage
    R = oracle.gemm_bf16(A, Bt)
    assert relfro(G, R) < 2.5e-3


@pytest.mark.parametrize("M,N,K", [(17, 33, 72), (300, 260, 136),
                                   (513, 1000, 1032), (256, 256, 8),
                                   (64, 2048, 520), (1500, 96, 200)])
def test_bf16_ragged(dev, M, N, K):
    A = gi.bf16_operand(10, M, K, std=K ** -0.5)
    Bt = gi.bf16_operand(11, N, K, std=K ** -0.5)
    C = tkg.gemm_bf16(_up(A, dev, torch.bfloat16), _up(Bt, dev, torch.bfloat16))
    check_bf16(_bf16_result(C), decode_bf16(A), decode_bf16(Bt), (M, N, K))


def test_bf16_k_zero_writes_zeros(dev):
    C = torch.full((40, 300), 7.0, dtype=torch.bfloat16, device=dev)
    A = torch.empty((40, 0), dtype=torch.bfloat16, device=dev)
    Bt = torch.empty((300, 0), dtype=torch.bfloat16, device=dev)
    tkg.gemm_bf16(A, Bt, out=C)
    assert not C.float().abs().sum().item()


def test_bf16_empty_output(dev):
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    Bt = torch.zeros((32, 64), dtype=torch.bfloat16, device=dev)
    assert tkg.gemm_bf16(A, Bt).shape == (0, 32)


def _sampled_bf16(dev, M, N, K, seed):
    A = gi.device.bf16_operand(seed, M, K, std=K ** -0.5, device=dev)
    Bt = gi.device.bf16_operand(seed + 1, N, K, std=K ** -0.5, device=dev)
    C = tkg.gemm_bf16(A, Bt)
    torch.cuda.synchronize()
    for (i0, j0) in sample_tiles(M, N, seed):
        a = decode_bf16(to_numpy_u16(A[i0:i0 + 64]))
        b = decode_bf16(to_numpy_u16(Bt[j0:j0 + 64]))
        G = _bf16_result(C[i0:i0 + 64, j0:j0 + 64])
        check_bf16(G, a, b, (M, N, K, i0, j0))


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 1024), (2048, 2048, 2048),
                                   (4096, 4096, 4096), (8192, 8192, 8192),
                                   (8192, 14336, 4096), (8192, 4096, 14336),
                                   (16384, 16384, 16384), (8192, 1024, 8192)])
def test_bf16_config_shapes_sampled(dev, M, N, K):
    # (8192, 1024, 8192): one GPU's N/8 share of the 8192^3 product, which
    # runs on 128 x 128 tiles (fewer 256 x 256 tiles than compute units)
    _sampled_bf16(dev, M, N, K, seed=100 + M % 997 + K % 13)


def test_bf16_launch_options_agree(dev):
    # persistent vs one-workgroup-per-tile, grouped vs row-major order,
    # XCD remap on/off: every output is computed by the same instruction
    # sequence, so results are identical bit for bit.
    M, N, K = 2048, 1536, 1024
    A = gi.device.bf16_operand(7, M, K, std=K ** -0.5, device=dev)
    Bt = gi.device.bf16_operand(8, N, K, std=K ** -0.5, device=dev)
    ref = tkg.gemm_bf16(A, Bt)
    for grid, gm, xr in [(10000, 0, 1), (0, 1, 1), (0, 3, 0), (64, 16, 1), (7, 8, 1),
                         (0, 8, 2), (0, 4, 2), (0, 16, 2), (24, 8, 2)]:
        C = torch.full_like(ref, float("nan"))
        st = tkg.tkg_gemm_ex(tkg.DTYPE_BF16, M, N, K, A, None, 1.0, Bt, None,
                             1.0, C, grid=grid, group_m=gm, xcd_remap=xr)
        assert st == 0
        assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), (grid, gm, xr)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_xcd_block_order_covers_every_tile(dev, dtype):
    # XCD-block order (xcd_remap 2) on full rounds: 16 x 16 tiles of 256 x 256
    # over grids of 64 and 256 workgroups, group_m 4 .. 16, plus a ragged last
    # band (M = 3000: 12 tile rows); a tile the map missed keeps its NaN fill,
    # a tile dealt twice would still match, so coverage plus bit equality
    # with the grouped order checks the map is a bijection.
    for M, N, K in [(4096, 4096, 256), (3000, 4096, 256)]:
        A, Bt, d, sa, sb = _dense_operands(dev, dtype, M, N, K, seed=41)
        ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, ref, xcd_remap=1) == 0
        for grid, gm in [(64, 16), (64, 4), (256, 8), (256, 16), (0, 16), (128, 8)]:
            C = torch.full_like(ref, float("nan"))
            assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, C, grid=grid,
                                   group_m=gm, xcd_remap=2) == 0
            assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), (M, grid, gm)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K", [(6144, 6144, 512), (4352, 4096, 1024), (6400, 6144, 256),
                                   (8448, 8448, 8192)])
def test_tail_quadrant_launch_agrees(dev, dtype, M, N, K):
    # a partial last round of 256 x 256 tiles runs as 128 x 128 quadrants in
    # a second launch; against the single launch (an explicit grid turns the
    # split off), bit for bit, every element written (NaN fill). 8448^2 x
    # 8192 bf16 also takes the large-operand ring and order.
    plan = tkg.plan_launch(tkg.DTYPE_BF16 if dtype == "bf16" else tkg.DTYPE_FP8, M, N, K)
    assert plan["tail_units"] > 0 and plan["units"] % plan["grid"] == 0, plan
    A, Bt, d, sa, sb = _dense_operands(dev, dtype, M, N, K, seed=43)
    ref = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, ref,
                           grid=plan["grid"]) == 0
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, C) == 0
    assert not torch.isnan(C.float()).any()
    assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), (M, N, K)
    if M * N * K <= 6144 * 6144 * 512:
        # the first tiles (first launch) and the last ones (quadrants)
        _check_dense(dtype, A[:256], Bt[:512], sa, sb, C[:256, :512].contiguous(), (M, N, K))
        _check_dense(dtype, A[-256:], Bt[-512:], sa, sb, C[-256:, -512:].contiguous(),
                     (M, N, K, "tail"))


def _dense_operands(dev, dtype, M, N, K, seed):
    if dtype == "bf16":
        A = gi.device.bf16_operand(seed, M, K, std=K ** -0.5, device=dev)
        Bt = gi.device.bf16_operand(seed + 1, N, K, std=K ** -0.5, device=dev)
        return A, Bt, tkg.DTYPE_BF16, 1.0, 1.0
    A, sa = gi.device.fp8_operand(seed, M, K, device=dev)
    Bt, sb = gi.device.fp8_operand(seed + 1, N, K, device=dev)
    return A, Bt, tkg.DTYPE_FP8, sa, sb


def _check_dense(dtype, A, Bt, sa, sb, C, what):
    a = to_numpy_u16(A) if dtype == "bf16" else to_numpy_u8(A)
    b = to_numpy_u16(Bt) if dtype == "bf16" else to_numpy_u8(Bt)
    G = _bf16_result(C)
    if dtype == "bf16":
        check_bf16(G, decode_bf16(a), decode_bf16(b), what)
    else:
        check_fp8_elementwise(G, a, sa, b, sb, what)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K,grid", [(1300, 700, 1088, 0), (1024, 768, 2048, 0),
                                        (1024, 768, 2048, 5), (520, 1280, 1664, 3)])
def test_kernel_variants_agree(dev, dtype, M, N, K, grid):
    # every compiled kernel configuration (LDS ring shape and depth, waves
    # per workgroup, MFMA block, swizzle on or off, interleaved, early-B or
    # ping-pong schedule) computes the same bits: on ragged edges (masked
    # instances), on whole tiles (unmasked instances) and with fewer
    # workgroups than tiles (the persistent loop crosses tiles and finishes)
    A, Bt, d, sa, sb = _dense_operands(dev, dtype, M, N, K, 3)
    nv = tkg.num_variants(d)
    assert nv >= 9
    outs = []
    for v in range(nv):
        C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=dev)
        assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, C, variant=v,
                               grid=grid) == 0, v
        outs.append(C)
    for v in range(1, nv):
        assert torch.equal(outs[v].view(torch.int16), outs[0].view(torch.int16)), (
            v, tkg.variant_info(d, v))
    _check_dense(dtype, A, Bt, sa, sb, outs[0], ("variants", M, N, K, grid))
    assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, outs[0], variant=nv) == -2


def test_fp8_block_shapes_at_long_k(dev):
    # At K = 16384 the fp32 sums are no longer exact. Configurations on
    # 32x32x64 blocks still agree with the default bit for bit; those on
    # 16x16x128 blocks round the accumulation at other points, so where a
    # sum lies next to a bf16 rounding midpoint the two can round to
    # neighbouring values. Each such element is checked, in both outputs,
    # against the oracle and its per-element bound.
    M = N = K = 16384
    A, Bt, d, sa, sb = _dense_operands(dev, "fp8", M, N, K, 11)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, ref) == 0
    assert tkg.variant_info(d, 0)["mfma_block"] == 32
    C = torch.empty_like(ref)
    seen = set()
    for v in range(1, tkg.num_variants(d)):
        assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, C, variant=v) == 0, v
        block = tkg.variant_info(d, v)["mfma_block"]
        seen.add(block)
        diff = (C.view(torch.int16) != ref.view(torch.int16)).nonzero().tolist()
        if block == 32:
            assert not diff, (v, len(diff))
            continue
        assert len(diff) <= 1000, (v, len(diff))
        for i, j in diff[:16]:
            a = to_numpy_u8(A[i:i + 1])
            b = to_numpy_u8(Bt[j:j + 1])
            R = oracle.gemm_fp8(a, sa, b, sb)
            bound = lowp_elem_bound(oracle.abs_gemm_f64(decode_e4m3(a) * float(sa),
                                                        decode_e4m3(b) * float(sb)), K)
            for G in (C, ref):
                g = _bf16_result(G[i:i + 1, j:j + 1].contiguous())
                assert np.all(np.abs(g - R) <= bound), (v, i, j)
    assert seen == {16, 32}
    _check_dense("fp8", A[:256], Bt[:512], sa, sb, ref[:256, :512].contiguous(),
                 ("fp8 long K", M, N, K))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_kernel_variants_k_zero(dev, dtype):
    # K = 0 writes zeros in every configuration (the ping-pong loop has no
    # k-step to hang the finish on)
    d = tkg.DTYPE_BF16 if dtype == "bf16" else tkg.DTYPE_FP8
    A = torch.empty((300, 0), dtype=torch.uint8, device=dev)
    for v in range(tkg.num_variants(d)):
        C = torch.full((300, 520), 5.0, dtype=torch.bfloat16, device=dev)
        assert tkg.tkg_gemm_ex(d, 300, 520, 0, A, None, 1.0, A, None, 1.0, C, variant=v) == 0
        assert torch.count_nonzero(C).item() == 0, v


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M,N,K", [(300, 260, 8192), (2048 + 40, 1024 + 8, 4096)])
def test_ragged_tiles_long_k(dev, dtype, M, N, K):
    # Regression: ragged M / N tiles with K a whole number of stages. The
    # rows past M (N) lie beyond the operands, so these launches must take
    # the masked instance, whose loads are bounds-checked per lane (the
    # scalar offset of the unmasked one is outside the bounds check). The
    # instance choice is checked here through tkg_launch_masked, the
    # results on every configuration.
    d = tkg.DTYPE_BF16 if dtype == "bf16" else tkg.DTYPE_FP8
    for v in (0, tkg.num_variants(d) - 1):
        assert tkg.launch_masked(d, M, N, K, v)
    A, Bt, d, sa, sb = _dense_operands(dev, dtype, M, N, K, 11)
    for v in range(tkg.num_variants(d)):
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, C, variant=v) == 0
        _check_dense(dtype, A, Bt, sa, sb, C, ("ragged long K", v))


def test_bf16_side_stream(dev):
    M = N = K = 512
    A = gi.bf16_operand(1, M, K)
    Bt = gi.bf16_operand(2, N, K)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Ad, Bd = _up(A, dev, torch.bfloat16), _up(Bt, dev, torch.bfloat16)
        C = tkg.gemm_bf16(Ad, Bd)
    s.synchronize()
    check_bf16(_bf16_result(C), decode_bf16(A), decode_bf16(Bt), "stream")


# ------------------------------------------------------------------ fp8

def test_fp8_identity_bit_exact(dev):
    M, K = 260, 256
    codes = gi.e4m3_codes(gi.normal(3, M, K) * 40)
    eye = np.zeros((K, K), np.uint8)
    np.fill_diagonal(eye, 0x38)                      # 1.0
    C = tkg.gemm_fp8(_up(codes, dev), 1.0, _up(eye, dev), 1.0)
    # every e4m3 value is exact in bf16 (incl. 448 = 0x7E, subnormals)
    assert np.array_equal(_bf16_result(C), decode_e4m3(codes))


def test_fp8_all_codes_decode(dev):
    # each of the 254 finite codes, once per row, against the identity
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    K = 256
    A = np.zeros((codes.size, K), np.uint8)
    A[np.arange(codes.size), np.arange(codes.size) % K] = codes
    eye = np.zeros((K, K), np.uint8)
    np.fill_diagonal(eye, 0x38)
    C = tkg.gemm_fp8(_up(A, dev), 1.0, _up(eye, dev), 1.0)
    G = _bf16_result(C)
    assert np.array_equal(G[np.arange(codes.size), np.arange(codes.size) % K],
                          decode_e4m3(codes))


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (300, 260, 144)])
def test_fp8_integers_bit_exact(dev, M, N, K):
    A = gi.e4m3_codes(gi.small_integers(6, M, K))
    Bt = gi.e4m3_codes(gi.small_integers(7, N, K))
    C = tkg.gemm_fp8(_up(A, dev), 1.0, _up(Bt, dev), 1.0)
    ref = round_to_bf16(oracle.gemm_fp8(A, 1.0, Bt, 1.0))
    assert np.array_equal(_bf16_result(C), ref)


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 260, 144),
                                   (1000, 513, 1040)])
def test_fp8_normal(dev, M, N, K):
    A, sa = gi.fp8_operand(20, M, K)
    Bt, sb = gi.fp8_operand(21, N, K)
    C = tkg.gemm_fp8(_up(A, dev), sa, _up(Bt, dev), sb)
    R = oracle.gemm_fp8(A, sa, Bt, sb)
    assert relfro(_bf16_result(C), R) <= LOWP_RELFRO


@pytest.mark.parametrize("M,N,K", [(8192, 8192, 8192), (16384, 16384, 16384),
                                   (8192, 1024, 8192)])
def test_fp8_config_shapes_sampled(dev, M, N, K):
    A, sa = gi.device.fp8_operand(30, M, K, device=dev)
    Bt, sb = gi.device.fp8_operand(31, N, K, device=dev)
    C = tkg.gemm_fp8(A, sa, Bt, sb)
    torch.cuda.synchronize()
    for (i0, j0) in sample_tiles(M, N, K):
        G = _bf16_result(C[i0:i0 + 64, j0:j0 + 64])
        check_fp8_elementwise(G, to_numpy_u8(A[i0:i0 + 64]), sa,
                              to_numpy_u8(Bt[j0:j0 + 64]), sb, (M, N, K, i0, j0))


# ----------------------------------------------------- block-scaled 4-bit

def _fp4_identity(K):
    codes = np.zeros((K, K), np.uint8)
    np.fill_diagonal(codes, 0x2)                     # 1.0
    return gi.pack_nibbles(codes), np.full((K, K // 16), 0x38, np.uint8)


def test_fp4_identity_bit_exact(dev):
    M, K = 272, 256
    Ap, As, _ = gi.fp4_quantize(gi.normal(40, M, K))
    Ip, Is = _fp4_identity(K)
    C = tkg.gemm_fp4_blockscaled(_up(Ap, dev), _up(As, dev), 1.0,
                                 _up(Ip, dev), _up(Is, dev), 1.0)
    # value x block scale is exact in bf16 (at most 6 significant bits)
    assert np.array_equal(_bf16_result(C), oracle.dequant_fp4_blockscaled(Ap, As))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 260, 192),
                                   (513, 700, 1088)])
def test_fp4_normal(dev, M, N, K):
    Ap, As, ta = gi.fp4_operand(41, M, K)
    Bp, Bs, tb = gi.fp4_operand(42, N, K)
    C = tkg.gemm_fp4_blockscaled(_up(Ap, dev), _up(As, dev), ta,
                                 _up(Bp, dev), _up(Bs, dev), tb)
    R = oracle.gemm_fp4_blockscaled(Ap, As, ta, Bp, Bs, tb)
    assert relfro(_bf16_result(C), R) <= LOWP_RELFRO


def test_fp4_integers_bit_exact(dev):
    # power-of-two block scales and tensor scales 1: exact accumulation
    M, N, K = 320, 288, 512
    g = np.random.default_rng(9)
    Ac = g.integers(0, 16, (M, K)).astype(np.uint8)
    Bc = g.integers(0, 16, (N, K)).astype(np.uint8)
    As = g.choice(np.array([0x30, 0x38, 0x40], np.uint8), (M, K // 16))
    Bs = g.choice(np.array([0x30, 0x38, 0x40], np.uint8), (N, K // 16))
    Ap, Bp = gi.pack_nibbles(Ac), gi.pack_nibbles(Bc)
    C = tkg.gemm_fp4_blockscaled(_up(Ap, dev), _up(As, dev), 1.0,
                                 _up(Bp, dev), _up(Bs, dev), 1.0)
    ref = round_to_bf16(oracle.gemm_fp4_blockscaled(Ap, As, 1.0, Bp, Bs, 1.0))
    assert np.array_equal(_bf16_result(C), ref)


def test_fp4_every_block_scale_code_bit_exact(dev):
    # Every finite e4m3 code as a block scale (subnormals, negatives, +-0,
    # 448) with every e2m1 code as a value, times the identity: value x
    # block scale has at most 6 significant bits, so C is the dequantized A
    # exactly (pins the in-register dequantization, scale byte selection
    # per lane half and block included).
    M, K = 256, 512
    g = np.random.default_rng(23)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    As = np.resize(finite, M * (K // 16)).reshape(M, K // 16)
    As = As[:, g.permutation(K // 16)]
    Ac = g.integers(0, 16, (M, K)).astype(np.uint8)
    Ap = gi.pack_nibbles(Ac)
    Ip, Is = _fp4_identity(K)
    C = tkg.gemm_fp4_blockscaled(_up(Ap, dev), _up(As, dev), 1.0,
                                 _up(Ip, dev), _up(Is, dev), 1.0)
    assert np.array_equal(_bf16_result(C), oracle.dequant_fp4_blockscaled(Ap, As))
    assert len(np.unique(As)) == 254


def test_fp4_signed_subnormal_and_zero_block_scales(dev):
    # Block scales of every kind the e4m3 format holds: negative (the sign
    # must reach the product), subnormal, +0 and -0, non-power-of-two
    # mantissas and the largest finite magnitude. Per-element bound: fp32
    # summation plus one bf16 rounding, at most 2^-8 (|A||B|)_ij here.
    M, N, K = 256, 320, 512
    g = np.random.default_rng(21)
    kinds = np.array([0x38, 0xB8, 0xBF, 0x3A, 0x01, 0x83, 0x07, 0x00, 0x80,
                      0x7E, 0xFE, 0x44, 0xC9], np.uint8)
    Ac = g.integers(0, 16, (M, K)).astype(np.uint8)
    Bc = g.integers(0, 16, (N, K)).astype(np.uint8)
    As = g.choice(kinds, (M, K // 16))
    Bs = g.choice(kinds, (N, K // 16))
    Ap, Bp = gi.pack_nibbles(Ac), gi.pack_nibbles(Bc)
    ta, tb = 0.75, 2.0 ** -12
    C = tkg.gemm_fp4_blockscaled(_up(Ap, dev), _up(As, dev), ta,
                                 _up(Bp, dev), _up(Bs, dev), tb)
    R = oracle.gemm_fp4_blockscaled(Ap, As, ta, Bp, Bs, tb)
    Ad = oracle.dequant_fp4_blockscaled(Ap, As)
    Bd = oracle.dequant_fp4_blockscaled(Bp, Bs)
    bound = 2.0 ** -8 * ta * tb * oracle.abs_gemm_f64(Ad, Bd)
    G = _bf16_result(C)
    assert np.all(np.abs(G - R) <= bound), float(np.max(np.abs(G - R) - bound))
    assert np.any(As & 0x80) and np.any(Bs & 0x80)
    assert relfro(G, R) <= 1e-2


def test_fp4_variants_agree(dev):
    M, N, K = 700, 1300, 1088
    Ap, As, ta = gi.fp4_operand(60, M, K)
    Bp, Bs, tb = gi.fp4_operand(61, N, K)
    args = [_up(Ap, dev), _up(As, dev), ta, _up(Bp, dev), _up(Bs, dev), tb]
    outs = []
    for v in range(2):
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        st = tkg.tkg_gemm_ex(tkg.DTYPE_FP4_BLOCKSCALED, M, N, K, args[0], args[1],
                             ta, args[3], args[4], tb, C, variant=v)
        assert st == 0
        outs.append(C)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    R = oracle.gemm_fp4_blockscaled(Ap, As, ta, Bp, Bs, tb)
    assert relfro(_bf16_result(outs[0]), R) <= LOWP_RELFRO


def test_fp4_xcd_block_order_agrees(dev):
    # 16 x 16 tiles of 256 x 256 over 64 workgroups in the XCD-block order
    # (full rounds re-dealt) against the default order, NaN-filled output
    M, N, K = 4096, 4096, 512
    Ap, As, ta = gi.device.fp4_operand(62, M, K, device=dev)
    Bp, Bs, tb = gi.device.fp4_operand(63, N, K, device=dev)
    outs = []
    for grid, gm, xr in ((0, 0, 1), (64, 16, 2), (64, 4, 2), (128, 8, 2)):
        C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
        st = tkg.tkg_gemm_ex(tkg.DTYPE_FP4_BLOCKSCALED, M, N, K, Ap, As, ta, Bp, Bs, tb, C,
                             grid=grid, group_m=gm, xcd_remap=xr)
        assert st == 0
        outs.append(C)
    for C in outs[1:]:
        assert torch.equal(C.view(torch.int16), outs[0].view(torch.int16))


@pytest.mark.parametrize("n", [16384, 65536])
def test_fp4_config_shapes_sampled(dev, n):
    Ap, As, ta = gi.device.fp4_operand(50, n, n, device=dev)
    Bp, Bs, tb = gi.device.fp4_operand(51, n, n, device=dev)
    C = tkg.gemm_fp4_blockscaled(Ap, As, ta, Bp, Bs, tb)
    torch.cuda.synchronize()
    tiles = sample_tiles(n, n, n, n_random=4 if n > 20000 else 8)
    for (i0, j0) in tiles:
        a, asc = to_numpy_u8(Ap[i0:i0 + 64]), to_numpy_u8(As[i0:i0 + 64])
        b, bsc = to_numpy_u8(Bp[j0:j0 + 64]), to_numpy_u8(Bs[j0:j0 + 64])
        R = oracle.gemm_fp4_blockscaled(a, asc, ta, b, bsc, tb)
        G = _bf16_result(C[i0:i0 + 64, j0:j0 + 64])
        assert relfro(G, R) <= LOWP_RELFRO, (n, i0, j0)
        # per element (the MX tests' form): fp32 sums of exact products
        absprod = float(ta) * float(tb) * oracle.abs_gemm_f64(
            oracle.dequant_fp4_blockscaled(a, asc), oracle.dequant_fp4_blockscaled(b, bsc))
        bound = lowp_elem_bound(absprod, n)
        assert np.all(np.abs(G - R) <= bound), (n, i0, j0, float(np.max(np.abs(G - R) - bound)))
    del C


def test_device_info_matches_the_device(dev):
    # the CU count behind the default grid is the one torch reports, and the
    # runtime's peak clock is set (MI355X: 2400 MHz)
    info = tkg.device_info()
    assert info["cus"] == torch.cuda.get_device_properties(dev).multi_processor_count
    assert 500.0 <= info["peak_clock_mhz"] <= 5000.0
