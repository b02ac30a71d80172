"""Seeded random shapes through the automatic launch: ragged tiles (masked
instance), whole tiles (unmasked), products that take the 128 x 128 tiles,
partial last rounds (tail quadrants in a second launch) and, for whole
rounds beyond the cache, the XCD-block order. Each product is checked on
sampled 64 x 64 tiles against the oracle element by element, and bit for
bit against the same product launched once in the grouped order."""
import numpy as np
import pytest
import torch

import gemm_inputs as gi
import gemm_inputs.device  # noqa: F401  (gi.device)
import tiled_dense_gemm_amd as tkg
from tests.parity import sample_tiles, to_numpy_u16, to_numpy_u8
from tests.test_gpu_parity import _bf16_result, check_bf16, check_fp8_elementwise
from tests.test_gpu_parity import dev  # noqa: F401  (the device fixture)
from oracle.formats import decode_bf16

# whole-tile edges that leave partial last rounds (272, 576, 600, 672 tiles
# of 256 x 256 on 256 compute units) and a few plain ones
WHOLE = [256, 1024, 4096, 4352, 4608, 5376, 6144, 6400, 6656, 7168]


def _case(i):
    rng = np.random.default_rng(9000 + i)
    kind = i % 4
    if kind == 0:      # ragged everywhere, any size
        M, N = (int(x) for x in rng.integers(1, 7000, 2))
    elif kind == 1:    # whole tiles
        M, N = (int(x) for x in rng.choice(WHOLE, 2))
    elif kind == 2:    # small: 128 x 128 tiles at two per CU
        M, N = (int(x) for x in rng.integers(1, 1500, 2))
    else:              # whole rows of tiles, ragged columns
        M, N = int(rng.choice(WHOLE)), int(rng.integers(100, 7000))
    # whole tiles take whole stages of K too (the unmasked instance)
    K = 128 * int(rng.integers(1, 24)) if kind == 1 else 16 * int(rng.integers(1, 160))
    return M, N, K


def _large(dtype):
    # operands beyond the 256 MB last-level cache (cache-sized bands in the
    # XCD-block order; bf16: the 5-slot ring) with a partial last round
    return (7168, 7168, 16384) if dtype == "bf16" else (7168, 7168, 32768)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", range(17))
def test_random_shape(dev, dtype, case):
    M, N, K = _case(case) if case < 16 else _large(dtype)
    seed = 700 + 31 * case + (dtype == "fp8")
    d = tkg.DTYPE_BF16 if dtype == "bf16" else tkg.DTYPE_FP8
    if dtype == "bf16":
        A = gi.device.bf16_operand(seed, M, K, std=K ** -0.5, device=dev)
        Bt = gi.device.bf16_operand(seed + 1, N, K, std=K ** -0.5, device=dev)
        sa = sb = 1.0
    else:
        A, sa = gi.device.fp8_operand(seed, M, K, device=dev)
        Bt, sb = gi.device.fp8_operand(seed + 1, N, K, device=dev)
    plan = tkg.plan_launch(d, M, N, K)
    what = (dtype, M, N, K, plan)
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, C) == 0, what
    ref = torch.full_like(C, float("nan"))
    assert tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, Bt, None, sb, ref, grid=plan["grid"],
                           group_m=8, xcd_remap=1) == 0, what
    torch.cuda.synchronize()
    assert not torch.isnan(C.float()).any(), what
    assert torch.equal(C.view(torch.int16), ref.view(torch.int16)), what
    for (i0, j0) in sample_tiles(M, N, seed, n_random=4):
        rows, cols = slice(i0, i0 + 64), slice(j0, j0 + 64)
        G = _bf16_result(C[rows, cols])
        if dtype == "bf16":
            check_bf16(G, decode_bf16(to_numpy_u16(A[rows])), decode_bf16(to_numpy_u16(Bt[cols])),
                       what + (i0, j0))
        else:
            check_fp8_elementwise(G, to_numpy_u8(A[rows]), sa, to_numpy_u8(Bt[cols]), sb,
                                  what + (i0, j0))


def test_random_shapes_cover_the_launch_forms():
    # host-side: the case list reaches every launch form at least once
    forms = set()
    for i in range(17):
        for d, name in ((tkg.DTYPE_BF16, "bf16"), (tkg.DTYPE_FP8, "fp8")):
            M, N, K = _case(i) if i < 16 else _large(name)
            p = tkg.plan_launch(d, M, N, K)
            forms.add(("small" if p["tile"] == 128 else "big",
                       bool(p["tail_units"]),
                       tkg.launch_masked(d, M, N, K, p["variant"])))
    assert ("small", False, True) in forms and ("big", False, True) in forms
    assert ("big", True, False) in forms and ("big", False, False) in forms
    p = tkg.plan_launch(tkg.DTYPE_BF16, *_large("bf16"))
    assert (p["variant"], p["xcd_remap"], p["tail_units"] > 0) == (18, 2, True)
    assert tkg.plan_launch(tkg.DTYPE_FP8, *_large("fp8"))["xcd_remap"] == 2
