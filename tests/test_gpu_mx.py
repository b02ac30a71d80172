"""GPU parity of the MX block-scaled products (gemm_mxfp4, gemm_mxfp8)
against the CPU oracle (oracle.gemm_mx), on the same bytes.

Tolerances: relative Frobenius <= 1e-2 against the fp64 product of the same
dequantized operands (the bf16 output rounding alone is ~1.7e-3), and per
element |G - R| <= 2^-8 (|A||B|)_ij (fp32 accumulation plus one bf16
rounding); structured operands whose products are exact in fp32 are compared
bit for bit with the oracle rounded to bf16.
"""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import gemm_inputs.device  # noqa: F401  (gi.device)
import oracle
import tiled_dense_gemm_amd as tkg
from oracle.formats import decode_bf16, round_to_bf16
from tests.parity import relfro, sample_tiles, to_numpy_u16, to_numpy_u8

pytestmark = pytest.mark.gpu

MX_RELFRO = 1e-2
ELEMS = ["e2m1", "e4m3"]
GEMM = {"e2m1": tkg.gemm_mxfp4, "e4m3": tkg.gemm_mxfp8}
DTYPE = {"e2m1": tkg.DTYPE_MXFP4, "e4m3": tkg.DTYPE_MXFP8}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need the HIP device"
    return torch.device("cuda:0")


def _up(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _result(C):
    return decode_bf16(to_numpy_u16(C))


def _check(G, Av, As, Bv, Bs, elem, what=""):
    R = oracle.gemm_mx(Av, As, Bv, Bs, elem)
    err = relfro(G, R)
    assert err <= MX_RELFRO, (what, err)
    bound = 2.0 ** -8 * oracle.abs_gemm_f64(oracle.dequant_mx(Av, As, elem),
                                            oracle.dequant_mx(Bv, Bs, elem))
    assert np.all(np.abs(G - R) <= bound + 1e-30), (what, float(np.max(np.abs(G - R) - bound)))


def _identity(elem, K):
    one = 0x2 if elem == "e2m1" else 0x38
    codes = np.zeros((K, K), np.uint8)
    np.fill_diagonal(codes, one)
    vals = gi.pack_nibbles(codes) if elem == "e2m1" else codes
    return vals, np.full((K, K // 32), 127, np.uint8)


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_identity_bit_exact(dev, elem):
    # element x 2^e has at most 4 significant bits: exact in bf16
    M, K = 288, 384
    Av, As = gi.mx_operand(70, M, K, elem)
    Iv, Is = _identity(elem, K)
    C = GEMM[elem](_up(Av, dev), _up(As, dev), _up(Iv, dev), _up(Is, dev))
    assert np.array_equal(_result(C), oracle.dequant_mx(Av, As, elem))


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 260, 384), (513, 700, 1152),
                                   (64, 1000, 128), (1, 1, 128)])
def test_mx_normal(dev, elem, M, N, K):
    Av, As = gi.mx_operand(71, M, K, elem)
    Bv, Bs = gi.mx_operand(72, N, K, elem)
    C = GEMM[elem](_up(Av, dev), _up(As, dev), _up(Bv, dev), _up(Bs, dev))
    _check(_result(C), Av, As, Bv, Bs, elem, (M, N, K))


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_integers_bit_exact(dev, elem):
    # integer-valued elements and scales 2^-1..2^1: every partial sum is an
    # exact fp32 value, so the result is the exactly rounded product
    M, N, K = 320, 288, 1024
    g = np.random.default_rng(31)
    if elem == "e2m1":
        pool = np.array([0, 2, 4, 5, 6, 7, 10, 12, 13, 14, 15], np.uint8)   # 0, +-1, +-2, +-3, +-4, +-6
        Ac, Bc = g.choice(pool, (M, K)), g.choice(pool, (N, K))
        Av, Bv = gi.pack_nibbles(Ac), gi.pack_nibbles(Bc)
    else:
        pool = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0xB8, 0xC0, 0xC4, 0xC8], np.uint8)
        Av, Bv = g.choice(pool, (M, K)), g.choice(pool, (N, K))
    As = g.choice(np.array([126, 127, 128], np.uint8), (M, K // 32))
    Bs = g.choice(np.array([126, 127, 128], np.uint8), (N, K // 32))
    C = GEMM[elem](_up(Av, dev), _up(As, dev), _up(Bv, dev), _up(Bs, dev))
    ref = round_to_bf16(oracle.gemm_mx(Av, As, Bv, Bs, elem))
    assert np.array_equal(_result(C), ref)


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_extreme_scales(dev, elem):
    # E8M0 across its range (2^-30 .. 2^30 here) on each block: scales are
    # applied per block of 32 inside the MFMA, not folded into the values
    M, N, K = 256, 256, 512
    g = np.random.default_rng(32)
    Av, _ = gi.mx_operand(73, M, K, elem)
    Bv, _ = gi.mx_operand(74, N, K, elem)
    As = g.integers(97, 158, (M, K // 32)).astype(np.uint8)
    Bs = g.integers(97, 158, (N, K // 32)).astype(np.uint8)
    C = GEMM[elem](_up(Av, dev), _up(As, dev), _up(Bv, dev), _up(Bs, dev))
    _check(_result(C), Av, As, Bv, Bs, elem, "extreme scales")


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_variants_agree(dev, elem):
    # the early-reads schedule (variant 1) reorders only LDS reads: the MFMA
    # sequence per accumulator is the same, so the bits are; shapes take
    # the wide-scale, narrow-scale and masked instances
    for M, N, K, seed in [(512, 768, 1024, 80), (512, 512, 640, 82), (300, 700, 1152, 84)]:
        Av, As = gi.mx_operand(seed, M, K, elem)
        Bv, Bs = gi.mx_operand(seed + 1, N, K, elem)
        args = [_up(Av, dev), _up(As, dev), _up(Bv, dev), _up(Bs, dev)]
        outs = []
        for v in (0, 1):
            C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
            assert tkg.tkg_gemm_ex(DTYPE[elem], M, N, K, args[0], args[1], 1.0, args[2],
                                   args[3], 1.0, C, variant=v) == 0
            outs.append(C)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), (M, N, K)
        if M == 512 and N == 768:
            R = oracle.gemm_mx(Av, As, Bv, Bs, elem)
            assert relfro(_result(outs[1]), R) <= MX_RELFRO


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_ex_output_scale_and_options(dev, elem):
    M, N, K = 700, 1300, 640
    Av, As = gi.mx_operand(75, M, K, elem)
    Bv, Bs = gi.mx_operand(76, N, K, elem)
    args = [_up(Av, dev), _up(As, dev), _up(Bv, dev), _up(Bs, dev)]
    outs = []
    for grid, gm, xr in ((0, 0, 1), (100000, 0, 1), (0, 1, 0), (16, 2, 2)):
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        st = tkg.tkg_gemm_ex(DTYPE[elem], M, N, K, args[0], args[1], 0.5, args[2], args[3],
                             0.25, C, grid=grid, group_m=gm, xcd_remap=xr)
        assert st == 0
        outs.append(C)
    for C in outs[1:]:
        assert torch.equal(C.view(torch.int16), outs[0].view(torch.int16))
    R = 0.125 * oracle.gemm_mx(Av, As, Bv, Bs, elem)
    assert relfro(_result(outs[0]), R) <= MX_RELFRO
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert tkg.tkg_gemm_ex(DTYPE[elem], M, N, K, args[0], args[1], 1.0, args[2], args[3],
                           1.0, C, variant=2) == tkg.STATUS["TKG_ERR_SHAPE"]


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("K", [512, 1536, 2048])
def test_mx_wide_scale_staging_across_tiles(dev, elem, K):
    # K % 512 == 0 stages scales 16 bytes per row (several stages at once,
    # two alternating LDS slots); a small grid makes every workgroup walk
    # several tiles, with an odd (K = 512, 1536) and an even (2048) number
    # of such loads per tile, so the slot parity carries across tiles
    M, N = 700, 1100
    Av, As = gi.mx_operand(79, M, K, elem)
    Bv, Bs = gi.mx_operand(80, N, K, elem)
    args = [_up(Av, dev), _up(As, dev), _up(Bv, dev), _up(Bs, dev)]
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    assert tkg.tkg_gemm_ex(DTYPE[elem], M, N, K, args[0], args[1], 1.0, args[2], args[3],
                           1.0, C, grid=5) == 0
    _check(_result(C), Av, As, Bv, Bs, elem, ("wide", K))


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_empty_k_gives_zeros(dev, elem):
    C = torch.full((64, 80), 3.0, dtype=torch.bfloat16, device=dev)
    e = torch.empty((64, 0), dtype=torch.uint8, device=dev)
    f = torch.empty((80, 0), dtype=torch.uint8, device=dev)
    GEMM[elem](e, e, f, f, out=C)
    assert torch.count_nonzero(C) == 0


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("n", [8192, 16384])
def test_mx_config_shapes_sampled(dev, elem, n):
    Av, As = gi.device.mx_operand(77, n, n, elem, device=dev)
    Bv, Bs = gi.device.mx_operand(78, n, n, elem, device=dev)
    C = GEMM[elem](Av, As, Bv, Bs)
    torch.cuda.synchronize()
    for (i0, j0) in sample_tiles(n, n, n, n_random=6):
        a, sa = to_numpy_u8(Av[i0:i0 + 64]), to_numpy_u8(As[i0:i0 + 64])
        b, sb = to_numpy_u8(Bv[j0:j0 + 64]), to_numpy_u8(Bs[j0:j0 + 64])
        R = oracle.gemm_mx(a, sa, b, sb, elem)
        assert relfro(_result(C[i0:i0 + 64, j0:j0 + 64]), R) <= MX_RELFRO, (n, i0, j0)
    del C


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_ragged_tiles_long_k(dev, elem):
    # Regression: ragged M and N with K a multiple of 512 (the wide scale
    # staging shape) must take the masked instance: rows past M / N lie
    # beyond the operands and only per-lane offsets are bounds-checked.
    M, N, K = 300, 260, 4096
    assert tkg.launch_masked(DTYPE[elem], M, N, K)
    assert not tkg.launch_masked(DTYPE[elem], 512, 256, K)
    Av, As = gi.mx_operand(90, M, K, elem)
    Bv, Bs = gi.mx_operand(91, N, K, elem)
    C = GEMM[elem](_up(Av, dev), _up(As, dev), _up(Bv, dev), _up(Bs, dev))
    _check(_result(C), Av, As, Bv, Bs, elem, ("ragged long K", M, N, K))
