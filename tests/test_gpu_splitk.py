"""GPU parity of the split-K products (tkg_gemm_splitk) against the CPU
oracle: K cut into ranges of whole stages, fp32 partial sums per range in a
caller workspace, added in range order by a second kernel. The tolerances
are those of the plain products (the sum order over K is unspecified);
integer-valued operands, whose partial sums are exact in fp32, are compared
bit for bit."""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import gemm_inputs.device  # noqa: F401  (gi.device)
import oracle
import tiled_dense_gemm_amd as tkg
from oracle.formats import decode_bf16, round_to_bf16
from tests.parity import relfro, to_numpy_u8, to_numpy_u16
from tests.test_gpu_parity import check_bf16, LOWP_RELFRO

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU parity tests need the HIP device"
    return torch.device("cuda:0")


def _res(C):
    return decode_bf16(to_numpy_u16(C))


@pytest.mark.parametrize("M,N,K,splits", [(1024, 1024, 16384, 0), (300, 260, 4096, 3),
                                          (64, 1000, 520, 0), (1, 1, 1024, 4),
                                          (130, 129, 2056, 5), (256, 256, 256, 64)])
def test_splitk_bf16(dev, M, N, K, splits):
    a = gi.bf16_operand(40, M, K)
    b = gi.bf16_operand(41, N, K)
    A = torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    Bt = torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
    C = tkg.gemm_splitk(A, Bt, splits=splits)
    assert tkg.splitk_count(tkg.DTYPE_BF16, M, N, K, splits) >= (2 if splits != 1 and K >= 1024 else 1)
    check_bf16(_res(C), decode_bf16(a), decode_bf16(b), ("splitk", M, N, K, splits))


@pytest.mark.parametrize("M,N,K,splits", [(512, 384, 8192, 0), (200, 300, 1040, 3)])
def test_splitk_fp8(dev, M, N, K, splits):
    a, sa = gi.fp8_operand(42, M, K)
    b, sb = gi.fp8_operand(43, N, K)
    C = tkg.gemm_splitk(torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev), sa, sb,
                        splits=splits)
    assert relfro(_res(C), oracle.gemm_fp8(a, sa, b, sb)) <= LOWP_RELFRO


def test_splitk_integers_bit_exact(dev):
    # integer entries in [-8, 8]: every partial and total sum is exact in
    # fp32, so the split result is the exactly rounded product
    M, N, K = 192, 320, 6144
    a = gi.small_integers(44, M, K)
    b = gi.small_integers(45, N, K)
    A = torch.from_numpy(gi.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
    Bt = torch.from_numpy(gi.bf16_bits(b).view(np.int16)).to(dev).view(torch.bfloat16)
    for s in (2, 7, 0):
        C = tkg.gemm_splitk(A, Bt, splits=s)
        assert np.array_equal(_res(C), round_to_bf16(oracle.gemm_f64(a, b))), s


def test_splitk_matches_plain_shape_rules_and_errors(dev):
    M, N, K = 128, 128, 4096
    A = gi.device.bf16_operand(46, M, K, device=dev)
    Bt = gi.device.bf16_operand(47, N, K, device=dev)
    need = tkg.splitk_workspace_size(tkg.DTYPE_BF16, M, N, K, 4)
    assert need == 4 * 128 * 128 * 4
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    small = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    st = tkg.lib.tkg_gemm_splitk(tkg.DTYPE_BF16, M, N, K, A.data_ptr(), 1.0, Bt.data_ptr(), 1.0,
                                 C.data_ptr(), small.data_ptr(), need - 16, 4, None)
    assert st == tkg.STATUS["TKG_ERR_WORKSPACE"]
    st = tkg.lib.tkg_gemm_splitk(tkg.DTYPE_BF16, M, N, K, A.data_ptr(), 1.0, Bt.data_ptr(), 1.0,
                                 C.data_ptr(), None, 0, 4, None)
    assert st == tkg.STATUS["TKG_ERR_WORKSPACE"]
    # one range: the plain product, no workspace
    assert tkg.splitk_workspace_size(tkg.DTYPE_BF16, M, N, K, 1) == 0
    C1 = tkg.gemm_splitk(A, Bt, splits=1)
    assert torch.equal(C1.view(torch.int16), tkg.gemm_bf16(A, Bt).view(torch.int16))
    # K = 0 gives zeros
    e = torch.empty((M, 0), dtype=torch.bfloat16, device=dev)
    f = torch.empty((N, 0), dtype=torch.bfloat16, device=dev)
    Z = torch.full((M, N), 2.0, dtype=torch.bfloat16, device=dev)
    tkg.gemm_splitk(e, f, splits=0, out=Z)
    assert torch.count_nonzero(Z) == 0


def test_splitk_repeated_calls_reuse_workspace(dev):
    # the workspace holds scratch only: a second, smaller call on the same
    # buffer gives its own product
    M, N, K = 256, 512, 8192
    A = gi.device.bf16_operand(48, M, K, std=K ** -0.5, device=dev)
    Bt = gi.device.bf16_operand(49, N, K, std=K ** -0.5, device=dev)
    ws = torch.empty(tkg.splitk_workspace_size(tkg.DTYPE_BF16, M, N, K, 8), dtype=torch.uint8,
                     device=dev)
    C = tkg.gemm_splitk(A, Bt, splits=8, workspace=ws)
    C2 = tkg.gemm_splitk(A[:100, :4096].contiguous(), Bt[:300, :4096].contiguous(), splits=3,
                         workspace=ws)
    torch.cuda.synchronize()
    a = to_numpy_u16(A).view(np.uint16); b = to_numpy_u16(Bt).view(np.uint16)
    check_bf16(_res(C), decode_bf16(a), decode_bf16(b), "first")
    check_bf16(_res(C2), decode_bf16(a[:100, :4096]), decode_bf16(b[:300, :4096]), "second")


def test_splitk_side_stream_owned_workspace(dev):
    # the binding allocates the workspace itself and runs on a side stream:
    # the block must stay reserved for that stream (record_stream) while an
    # allocation on the current stream follows at once
    M, N, K = 512, 512, 16384
    a = gi.bf16_operand(50, M, K, std=K ** -0.5)
    b = gi.bf16_operand(51, N, K, std=K ** -0.5)
    A = torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    Bt = torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    C.record_stream(s)
    need = tkg.splitk_workspace_size(tkg.DTYPE_BF16, M, N, K, 8)
    for _ in range(3):
        tkg.gemm_splitk(A, Bt, splits=8, out=C, stream=s)
        # same-size block on the current stream, written right away
        junk = torch.empty(need, dtype=torch.uint8, device=dev)
        junk.fill_(0x7F)
    s.synchronize()
    torch.cuda.synchronize()
    check_bf16(_res(C), decode_bf16(a), decode_bf16(b), "side stream")
