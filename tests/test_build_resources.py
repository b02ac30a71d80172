"""Register and LDS use of the compiled kernels, from the compiler's
kernel-resource-usage report that the build writes
(tiled_dense_gemm_amd/_build_obj/kernel_resources.json). Guards against a
change that pushes the default kernels into register spills in their main
loop (a stray live value once cost the fp8 kernel 60% of its rate): the
kernels that carry the default paths may spill at most a few registers
(their finish code), and every kernel fits the LDS."""
import json
import os
import re

import pytest

REPORT = os.path.join(os.path.dirname(os.path.dirname(__file__)), "tiled_dense_gemm_amd",
                      "_build_obj", "kernel_resources.json")

# template-argument prefixes of the default-path kernels (operand type, K
# bytes per stage, slots, wave columns, loaders, MFMA block, tile edge,
# workgroups per CU, swizzle, schedule, split-K)
DEFAULT_PATHS = [
    "gemm_dense_kernelILi0ELi128ELi4ELi4ELi1ELi16ELi256ELi1ELi1ELi0ELb0E",   # bf16
    "gemm_dense_kernelILi1ELi128ELi4ELi4ELi1ELi32ELi256ELi1ELi1ELi0ELb0E",   # fp8
    "gemm_dense_kernelILi0ELi128ELi4ELi2ELi0ELi16ELi128ELi2ELi1ELi0ELb",     # bf16 128x128 (+split-K)
    "gemm_dense_kernelILi1ELi128ELi4ELi2ELi0ELi16ELi128ELi2ELi1ELi0ELb",     # fp8 128x128 (+split-K)
    "gemm_fp4_kernelILi2E",
    "gemm_mx_kernel",
    "attn_fwd_kernel",
]


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(REPORT):
        pytest.skip("no build report (run tiled_dense_gemm_amd/_build.py)")
    return json.load(open(REPORT))


def test_default_kernels_barely_spill(report):
    for prefix in DEFAULT_PATHS:
        hits = {k: v for k, v in report.items() if prefix in k}
        assert hits, prefix
        for k, v in hits.items():
            assert v["VGPRs Spill"] <= 16, (k, v)
            assert v["ScratchSize"] <= 64, (k, v)


def test_every_kernel_fits_the_lds(report):
    for k, v in report.items():
        if "gemm" in k or "attn" in k:
            assert v["LDS Size"] <= 160 * 1024, (k, v)
        m = re.search(r"gemm_dense_kernelILi\d+ELi\d+ELi\d+ELi\d+ELi\d+ELi\d+ELi\d+ELi(\d+)E", k)
        if m and int(m.group(1)) == 2:   # two workgroups per CU share its LDS
            assert v["LDS Size"] <= 80 * 1024, (k, v)


def test_attention_occupancy(report):
    # (D, waves per workgroup, slots, waves per SIMD): the registers allow
    # the waves per SIMD the configuration asks for, and the LDS of the
    # workgroups resident on a CU fits
    import re
    hits = {k: v for k, v in report.items() if "attn_fwd_kernel" in k}
    assert len(hits) == 4
    for k, v in hits.items():
        m = re.search(r"attn_fwd_kernelILi(\d+)ELb(\d)ELi(\d+)ELi(\d+)ELi(\d+)ELb(\d)E", k)
        assert m, k
        waves, occ = int(m.group(3)), int(m.group(5))
        assert v["Occupancy"] >= occ, (k, v)
        assert v["LDS Size"] * (occ * 4 // waves) <= 160 * 1024, (k, v)
