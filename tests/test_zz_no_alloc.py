"""The allocation-free split-K entry point (tkg_gemm_splitk_noalloc)
against the split-K entry point with a caller workspace (tkg_gemm_splitk):
both run the same kernels with the same plan, so the results agree bit for
bit, and both meet the oracle tolerances of the plain products. Two calls
in a row share the library's device scratch; the second, smaller one must
give its own product. A plan larger than the scratch is rejected before
anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import gemm_inputs.device  # noqa: F401  (gi.device)
import oracle
import tiled_dense_gemm_amd as tkg
from oracle.formats import decode_bf16
from tests.parity import relfro, to_numpy_u8, to_numpy_u16
from tests.test_gpu_parity import check_bf16, check_fp8_elementwise

pytestmark = pytest.mark.gpu
L = tkg.lib


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "needs the HIP device"
    return torch.device("cuda:0")


def _noalloc(d, M, N, K, A, sa, Bt, sb, C, splits):
    return L.tkg_gemm_splitk_noalloc(d, M, N, K, A.data_ptr(), sa, Bt.data_ptr(), sb,
                                     C.data_ptr(), splits, None)


def _with_workspace(d, M, N, K, A, sa, Bt, sb, C, splits):
    need = tkg.splitk_workspace_size(d, M, N, K, splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=A.device)
    st = L.tkg_gemm_splitk(d, M, N, K, A.data_ptr(), sa, Bt.data_ptr(), sb, C.data_ptr(),
                           ws.data_ptr(), need, splits, None)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_matches_workspace_entry_two_calls(dev, dtype):
    # first call: 1024 x 1024 x 16384, automatic plan (8 ranges of 64 tiles:
    # 32 MiB of partials, the whole scratch); second, smaller: 300 x 260 x
    # 4096 in 3 ranges (ragged tiles), reusing the scratch
    d = tkg.DTYPE_BF16 if dtype == "bf16" else tkg.DTYPE_FP8
    for (M, N, K, splits, seed) in [(1024, 1024, 16384, 0, 60), (300, 260, 4096, 3, 62)]:
        if dtype == "bf16":
            A = gi.device.bf16_operand(seed, M, K, std=K ** -0.5, device=dev)
            Bt = gi.device.bf16_operand(seed + 1, N, K, std=K ** -0.5, device=dev)
            sa = sb = 1.0
        else:
            A, sa = gi.device.fp8_operand(seed, M, K, device=dev)
            Bt, sb = gi.device.fp8_operand(seed + 1, N, K, device=dev)
        assert tkg.splitk_count(d, M, N, K, splits) > 1
        assert tkg.splitk_workspace_size(d, M, N, K, splits) <= tkg.NOALLOC_SCRATCH_BYTES
        C0 = torch.full((M, N), 9.0, dtype=torch.bfloat16, device=dev)
        C1 = torch.full((M, N), -9.0, dtype=torch.bfloat16, device=dev)
        assert _noalloc(d, M, N, K, A, sa, Bt, sb, C0, splits) == 0
        torch.cuda.synchronize()
        assert _with_workspace(d, M, N, K, A, sa, Bt, sb, C1, splits) == 0
        assert torch.equal(C0.view(torch.int16), C1.view(torch.int16)), (M, N, K)
        G = decode_bf16(to_numpy_u16(C0))
        if dtype == "bf16":
            check_bf16(G, decode_bf16(to_numpy_u16(A)), decode_bf16(to_numpy_u16(Bt)),
                       ("noalloc", M, N, K))
        else:
            check_fp8_elementwise(G, to_numpy_u8(A), sa, to_numpy_u8(Bt), sb,
                                  ("noalloc", M, N, K))


def test_noalloc_binding_and_limits(dev):
    M, N, K = 256, 384, 8192
    A = gi.device.bf16_operand(70, M, K, std=K ** -0.5, device=dev)
    Bt = gi.device.bf16_operand(71, N, K, std=K ** -0.5, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    tkg.gemm_splitk_noalloc(A, Bt, C, splits=4)
    ref = tkg.gemm_splitk(A, Bt, splits=4)
    torch.cuda.synchronize()
    assert torch.equal(C.view(torch.int16), ref.view(torch.int16))
    # one range runs the plain product (no scratch)
    C2 = torch.empty_like(C)
    tkg.gemm_splitk_noalloc(A, Bt, C2, splits=1)
    assert torch.equal(C2.view(torch.int16), tkg.gemm_bf16(A, Bt).view(torch.int16))
    # a plan larger than the scratch is refused and leaves C untouched:
    # 2048 x 2048 x 8192 in 64 ranges needs 256 tiles x 64 x 64 KiB = 1 GiB
    Mb = Nb = 2048
    assert tkg.splitk_workspace_size(tkg.DTYPE_BF16, Mb, Nb, 8192, 64) > tkg.NOALLOC_SCRATCH_BYTES
    Ab = torch.zeros((Mb, 8192), dtype=torch.bfloat16, device=dev)
    Cb = torch.full((Mb, Nb), 7.0, dtype=torch.bfloat16, device=dev)
    st = L.tkg_gemm_splitk_noalloc(tkg.DTYPE_BF16, Mb, Nb, 8192, Ab.data_ptr(), 1.0,
                                   Ab.data_ptr(), 1.0, Cb.data_ptr(), 64, None)
    assert st == tkg.STATUS["TKG_ERR_WORKSPACE"]
    torch.cuda.synchronize()
    assert bool((Cb == 7.0).all())
    # argument errors as the workspace entry point
    assert L.tkg_gemm_splitk_noalloc(tkg.DTYPE_BF16, M, N, 12, A.data_ptr(), 1.0,
                                     Bt.data_ptr(), 1.0, C.data_ptr(), 0, None) == \
        tkg.STATUS["TKG_ERR_SHAPE"]
    assert L.tkg_gemm_splitk_noalloc(9, M, N, K, A.data_ptr(), 1.0, Bt.data_ptr(), 1.0,
                                     C.data_ptr(), 0, None) == tkg.STATUS["TKG_ERR_SHAPE"]
