"""The C-ABI library: loads without a GPU, exports every function that
include/tkg.h declares, and rejects invalid arguments with the documented
status before touching any device (these calls never reach the GPU)."""
import ctypes
import os
import re

import pytest

import tiled_dense_gemm_amd as tkg

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tkg.h")
S = tkg.STATUS


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"defined"})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gemm_bf16", "gemm_fp8", "gemm_fp4_blockscaled", "gemm_mxfp4", "gemm_mxfp8",
              "tkg_status_string", "tkg_gemm_ex", "tkg_attention_fwd", "tkg_attn_lds_offsets"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(tkg.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    for name, v in S.items():
        assert tkg.tkg_status_string(v).startswith(name)
    assert "unknown" in tkg.tkg_status_string(12345)


A16, B16, C16 = 4096, 8192, 12288   # 16-byte aligned fake addresses
L = tkg.lib


@pytest.mark.parametrize("call,want", [
    # negative or unsupported sizes
    (lambda: L.gemm_bf16(-1, 8, 8, A16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_bf16(8, -1, 8, A16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_bf16(8, 8, -8, A16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_bf16(8, 8, 12, A16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_bf16(8, 8, 1 << 23, A16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_bf16(1 << 31, 8, 8, A16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_fp8(8, 8, 24, A16, 1.0, B16, 1.0, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_fp4_blockscaled(8, 8, 96, A16, A16, 1.0, B16, B16, 1.0, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_gemm_ex(7, 8, 8, 8, A16, None, 1.0, B16, None, 1.0, C16, None, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_mxfp4(8, 8, 64, A16, A16, B16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_mxfp8(8, 8, 96, A16, A16, B16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_mxfp4(8, 8, 128, A16, None, B16, B16, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_mxfp8(8, 8, 128, A16, A16, B16, None, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_mxfp4(8, 8, 128, A16, A16 + 4, B16, B16, C16, None), S["TKG_ERR_ALIGN"]),
    (lambda: L.gemm_mxfp8(0, 0, 128, None, None, None, None, None, None), S["TKG_OK"]),
    # the largest K of each format passes the shape check (and stops at the
    # null pointer); one K granule more is rejected
    (lambda: L.gemm_bf16(8, 8, 4194296, None, B16, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_bf16(8, 8, 4194304, None, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_fp8(8, 8, 8388592, None, 1.0, B16, 1.0, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_fp8(8, 8, 8388608, None, 1.0, B16, 1.0, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_fp4_blockscaled(8, 8, 16777152, None, A16, 1.0, B16, B16, 1.0, C16, None),
     S["TKG_ERR_NULL"]),
    (lambda: L.gemm_fp4_blockscaled(8, 8, 16777216, None, A16, 1.0, B16, B16, 1.0, C16, None),
     S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_mxfp4(8, 8, 16777088, None, A16, B16, B16, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_mxfp4(8, 8, 16777216, None, A16, B16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.gemm_mxfp8(8, 8, 8388480, None, A16, B16, B16, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_mxfp8(8, 8, 8388608, None, A16, B16, B16, C16, None), S["TKG_ERR_SHAPE"]),
    # null pointers
    (lambda: L.gemm_bf16(8, 8, 8, None, B16, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_bf16(8, 8, 8, A16, None, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_bf16(8, 8, 8, A16, B16, None, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_fp8(8, 8, 16, A16, 1.0, None, 1.0, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_fp4_blockscaled(8, 8, 64, A16, None, 1.0, B16, B16, 1.0, C16, None), S["TKG_ERR_NULL"]),
    (lambda: L.gemm_fp4_blockscaled(8, 8, 64, A16, A16, 1.0, B16, None, 1.0, C16, None), S["TKG_ERR_NULL"]),
    # misaligned pointers
    (lambda: L.gemm_bf16(8, 8, 8, A16 + 2, B16, C16, None), S["TKG_ERR_ALIGN"]),
    (lambda: L.gemm_bf16(8, 8, 8, A16, B16 + 8, C16, None), S["TKG_ERR_ALIGN"]),
    (lambda: L.gemm_bf16(8, 8, 8, A16, B16, C16 + 4, None), S["TKG_ERR_ALIGN"]),
    (lambda: L.gemm_fp8(8, 8, 16, A16 + 1, 1.0, B16, 1.0, C16, None), S["TKG_ERR_ALIGN"]),
    (lambda: L.gemm_fp4_blockscaled(8, 8, 64, A16, A16 + 4, 1.0, B16, B16, 1.0, C16, None), S["TKG_ERR_ALIGN"]),
    # empty products succeed without reading any pointer
    (lambda: L.gemm_bf16(0, 8, 8, None, None, None, None), S["TKG_OK"]),
    (lambda: L.gemm_fp8(8, 0, 16, None, 1.0, None, 1.0, None, None), S["TKG_OK"]),
    (lambda: L.gemm_fp4_blockscaled(0, 0, 64, None, None, 1.0, None, None, 1.0, None, None), S["TKG_OK"]),
    # attention forward: (Q, K, V, O, lse, B, Hq, Hkv, Nq, Nk, D, scale, causal, stream)
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, 8, 96, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 3, 2, 8, 8, 64, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 0, 8, 8, 64, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, 9, 64, 0.1, 1, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, -1, 2, 2, 8, 8, 64, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, 0, 64, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 1 << 24, 8, 64, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    # sizes whose byte counts overflow 64 bits are rejected, not wrapped
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, (1 << 62) + 8, 128, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 1 << 62, 8, 64, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    # the most keys one head may hold (Nk * 2D < 2^31) passes the size checks
    (lambda: L.tkg_attention_fwd(None, None, None, None, None, 1, 2, 2, 8, (2**31 - 1) // 256, 128, 0.1, 0, None), S["TKG_ERR_NULL"]),
    (lambda: L.tkg_attention_fwd(None, None, None, None, None, 1, 2, 2, 8, (2**31 - 1) // 256 + 1, 128, 0.1, 0, None), S["TKG_ERR_SHAPE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, 8, 64, 0.0, 0, None), S["TKG_ERR_VALUE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, 8, 64, -1.0, 0, None), S["TKG_ERR_VALUE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, 8, 64, float("inf"), 0, None), S["TKG_ERR_VALUE"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, None, 1, 2, 2, 8, 8, 64, float("nan"), 0, None), S["TKG_ERR_VALUE"]),
    (lambda: L.tkg_attention_fwd(A16, None, C16, A16, None, 1, 2, 2, 8, 8, 64, 0.1, 0, None), S["TKG_ERR_NULL"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, None, None, 1, 2, 2, 8, 8, 64, 0.1, 0, None), S["TKG_ERR_NULL"]),
    (lambda: L.tkg_attention_fwd(A16 + 8, B16, C16, A16, None, 1, 2, 2, 8, 8, 64, 0.1, 0, None), S["TKG_ERR_ALIGN"]),
    (lambda: L.tkg_attention_fwd(A16, B16, C16, A16, C16 + 2, 1, 2, 2, 8, 8, 64, 0.1, 0, None), S["TKG_ERR_ALIGN"]),
    (lambda: L.tkg_attention_fwd(None, None, None, None, None, 0, 2, 2, 8, 8, 64, 0.1, 0, None), S["TKG_OK"]),
    (lambda: L.tkg_attention_fwd(None, None, None, None, None, 1, 2, 2, 0, 8, 128, 0.1, 0, None), S["TKG_OK"]),
    (lambda: L.tkg_attention_fwd(None, None, None, None, None, 1, 0, 0, 8, 8, 64, 0.1, 0, None), S["TKG_OK"]),
])
def test_argument_errors(call, want):
    assert call() == want


def test_splitk_plan_and_errors():
    # explicit range counts need no device: the plan is host arithmetic
    # (stages of 128 K-bytes, ranges of whole two-stage chunks, at most 64)
    bf, f8 = tkg.DTYPE_BF16, tkg.DTYPE_FP8
    assert tkg.splitk_count(bf, 1024, 1024, 16384, 8) == 8
    assert tkg.splitk_count(bf, 1024, 1024, 1024, 64) == 8      # 8 two-stage chunks of K
    assert tkg.splitk_count(f8, 512, 512, 1040, 3) == 3         # chunks 5 -> ranges of 2, 2, 1
    assert tkg.splitk_count(bf, 100, 100, 0, 4) == 1            # empty K: the plain product
    assert tkg.splitk_workspace_size(bf, 1024, 1024, 16384, 8) == 64 * 8 * 128 * 128 * 4
    assert tkg.splitk_workspace_size(bf, 1000, 130, 4096, 2) == 8 * 2 * 2 * 128 * 128 * 4
    assert tkg.splitk_workspace_size(bf, 512, 512, 4096, 1) == 0
    assert tkg.splitk_workspace_size(bf, 0, 512, 4096, 4) == 0
    assert L.tkg_gemm_splitk_workspace_size(2, 8, 8, 64, 2) == S["TKG_ERR_SHAPE"]
    assert L.tkg_gemm_splitk_workspace_size(bf, 8, 8, 12, 2) == S["TKG_ERR_SHAPE"]
    assert L.tkg_gemm_splitk_count(bf, 8, 8, 64, -1) == S["TKG_ERR_SHAPE"]
    # a needed workspace that is missing or short is refused before any launch
    assert L.tkg_gemm_splitk(bf, 256, 256, 8192, A16, 1.0, B16, 1.0, C16, None, 0, 4,
                             None) == S["TKG_ERR_WORKSPACE"]
    need = tkg.splitk_workspace_size(bf, 256, 256, 8192, 4)
    assert L.tkg_gemm_splitk(bf, 256, 256, 8192, A16, 1.0, B16, 1.0, C16, A16, need - 1, 4,
                             None) == S["TKG_ERR_WORKSPACE"]
    assert L.tkg_gemm_splitk(bf, 256, 256, 8192, A16, 1.0, B16, 1.0, C16, A16 + 8, need, 4,
                             None) == S["TKG_ERR_ALIGN"]
    assert L.tkg_gemm_splitk(bf, 256, 256, 8192, None, 1.0, B16, 1.0, C16, A16, need, 4,
                             None) == S["TKG_ERR_NULL"]
    assert L.tkg_gemm_splitk(2, 256, 256, 8192, A16, 1.0, B16, 1.0, C16, A16, need, 4,
                             None) == S["TKG_ERR_SHAPE"]
    assert L.tkg_gemm_splitk(bf, 0, 256, 8192, None, 1.0, None, 1.0, None, None, 0, 4,
                             None) == S["TKG_OK"]


def test_lds_introspection_errors():
    buf = (ctypes.c_uint32 * 64)()
    assert L.tkg_lds_fragment_offsets(0, 99, 0, 0, buf) == S["TKG_ERR_SHAPE"]
    assert L.tkg_lds_fragment_offsets(0, 0, 0, 0, None) == S["TKG_ERR_NULL"]
    assert L.tkg_lds_row_bytes(9) == S["TKG_ERR_SHAPE"]


def test_build_script_loads_without_its_package():
    # __graft_entry__.build() must work when libtkg.so is missing or stale,
    # so the build script may not import the package (which loads the
    # library on import).
    import ast
    import importlib.util
    path = os.path.join(os.path.dirname(tkg.__file__), "_build.py")
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.ImportFrom):
            assert node.level == 0 and not (node.module or "").startswith("tiled_dense_gemm_amd")
        if isinstance(node, ast.Import):
            assert all(not a.name.startswith("tiled_dense_gemm_amd") for a in node.names)
    spec = importlib.util.spec_from_file_location("tkg_build_probe", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert callable(mod.build) and mod.LIB.endswith("libtkg.so")


def test_splitk_count_rejects_oversized_k():
    # K beyond the product's limit is a shape error in the count query too
    # (it used to divide by a split length that overflowed to zero)
    for k in (1 << 31, 1 << 23, 4194312):
        assert L.tkg_gemm_splitk_count(0, 256, 256, k, 1) == S["TKG_ERR_SHAPE"]
    assert L.tkg_gemm_splitk_count(1, 256, 256, 1 << 24, 0) == S["TKG_ERR_SHAPE"]
    assert L.tkg_gemm_splitk_count(0, 256, 256, 12, 1) == S["TKG_ERR_SHAPE"]   # K % 8
    assert L.tkg_gemm_splitk_count(0, -1, 256, 1024, 1) == S["TKG_ERR_SHAPE"]
    assert L.tkg_gemm_splitk_count(0, 256, 256, 4194296, 1) == 1


def test_variant_table():
    # every dtype reports its configurations; the defaults are the measured
    # ones, and the ablation entries differ from the default in one field
    assert tkg.num_variants(tkg.DTYPE_BF16) == 20
    assert tkg.num_variants(tkg.DTYPE_FP8) == 14
    assert tkg.num_variants(tkg.DTYPE_FP4_BLOCKSCALED) == 2
    assert tkg.num_variants(tkg.DTYPE_MXFP4) == tkg.num_variants(tkg.DTYPE_MXFP8) == 2
    assert tkg.variant_info(tkg.DTYPE_MXFP4, 1)["schedule_name"] == "early reads"
    for d in (tkg.DTYPE_BF16, tkg.DTYPE_FP8):
        v0 = tkg.variant_info(d, 0)
        assert (v0["stage_kbytes"], v0["slots"], v0["waves"], v0["load_waves"], v0["tile"],
                v0["swizzle"]) == (128, 4, 8, 4, 256, 1)
        # bf16 defaults to early reads, fp8 to the interleaved schedule
        assert v0["schedule_name"] == ("early reads" if d == tkg.DTYPE_BF16 else "interleaved")
        small = tkg.variant_info(d, 4)
        assert small["tile"] == 128 and small["per_cu"] == 2
        swz = tkg.variant_info(d, 6)
        assert swz["swizzle"] == 0 and {k: v for k, v in swz.items() if k != "swizzle"} == \
            {k: v for k, v in v0.items() if k != "swizzle"}
        assert tkg.variant_info(d, 7)["schedule_name"] == "early B release"
        assert tkg.variant_info(d, 8)["schedule_name"] == "ping-pong"
        # the last entry: the small-tile configuration on the interleaved
        # schedule, the one before it the 5-slot ring with early reads
        last, small = tkg.variant_info(d, tkg.num_variants(d) - 1), tkg.variant_info(d, 4)
        assert last["schedule_name"] == "interleaved" and small["schedule_name"] == "early reads"
        assert {k: v for k, v in last.items() if not k.startswith("schedule")} == \
            {k: v for k, v in small.items() if not k.startswith("schedule")}
        five = tkg.variant_info(d, tkg.num_variants(d) - 2)
        assert (five["schedule_name"], five["slots"]) == ("early reads", 5)
        n = tkg.num_variants(d)
        assert L.tkg_variant_info(d, n, None) == S["TKG_ERR_SHAPE"]
        assert L.tkg_variant_info(d, -1, None) == S["TKG_ERR_SHAPE"]
    # the fp8 configurations on 16x16x128 blocks, the ones whose sums can
    # round differently from the default's 32x32x64 at long K
    assert [v for v in range(tkg.num_variants(tkg.DTYPE_FP8))
            if tkg.variant_info(tkg.DTYPE_FP8, v)["mfma_block"] == 16] == [2, 4, 5, 10, 13]
    # bf16 17 is the interleaved schedule, otherwise the default
    v17, v0 = tkg.variant_info(tkg.DTYPE_BF16, 17), tkg.variant_info(tkg.DTYPE_BF16, 0)
    assert v17["schedule_name"] == "interleaved"
    assert {k: v for k, v in v17.items() if not k.startswith("schedule")} == \
        {k: v for k, v in v0.items() if not k.startswith("schedule")}
    # the ring-depth sweep: 64-byte stages in rings of 1 .. 5 stages
    depth = [tkg.variant_info(tkg.DTYPE_BF16, v) for v in range(10, 15)]
    assert [d["slots"] // 2 for d in depth] == [1, 2, 3, 4, 5]
    assert {d["stage_kbytes"] for d in depth} == {64}
    assert L.tkg_variant_info(9, 0, None) == S["TKG_ERR_SHAPE"]


@pytest.mark.parametrize("dtype", [0, 1])
def test_masked_instance_choice(dtype):
    # the unmasked instance (part of each load's offset in the scalar offset,
    # which the buffer bounds check does not cover) runs only on whole tiles
    # with every stage inside K
    eb = 2 if dtype == 0 else 1
    for v in range(tkg.num_variants(dtype)):
        info = tkg.variant_info(dtype, v)
        bt, trip = info["tile"], 2 * info["stage_kbytes"] // eb   # K elements
        assert not tkg.launch_masked(dtype, 8 * bt, 4 * bt, 4 * trip, v), v
        assert tkg.launch_masked(dtype, 8 * bt - 1, 4 * bt, 4 * trip, v), v
        assert tkg.launch_masked(dtype, 8 * bt, 4 * bt + 16, 4 * trip, v), v
        assert tkg.launch_masked(dtype, 300, 260, 8192, v), v
        assert tkg.launch_masked(dtype, 8 * bt, 4 * bt, 4 * trip + 16, v), v
    assert tkg.launch_masked(tkg.DTYPE_FP4_BLOCKSCALED, 8192, 8192, 8192)
    assert not tkg.launch_masked(tkg.DTYPE_MXFP4, 8192, 8192, 8192)
    assert tkg.launch_masked(tkg.DTYPE_MXFP4, 300, 8192, 8192)
    assert tkg.launch_masked(tkg.DTYPE_MXFP8, 8192, 8200, 8192)
    # a stage is 128 bytes of values: an MXFP4 row of 8320 elements ends
    # mid-stage, an MXFP8 one does not
    assert tkg.launch_masked(tkg.DTYPE_MXFP4, 8192, 8192, 8320)
    assert not tkg.launch_masked(tkg.DTYPE_MXFP8, 8192, 8192, 8320)
    assert L.tkg_launch_masked(0, -1, 8, 8, 0) == S["TKG_ERR_SHAPE"]
    assert L.tkg_launch_masked(0, 8, 8, 8, 99) == S["TKG_ERR_SHAPE"]


def test_plan_launch_policy():
    # the launch tkg_gemm_ex makes, on the host: variant 0 resolved by tile
    # count and by operand size against the 256 MB last-level cache, and
    # the tile order (cache-sized bands in the XCD-block order) for
    # products whose A and B exceed that cache
    P = tkg.plan_launch
    bf, f8 = tkg.DTYPE_BF16, tkg.DTYPE_FP8
    one = dict(units=1024, tail_variant=-1, tail_units=0, tail_grid=0)
    assert P(bf, 8192, 8192, 8192) == dict(variant=0, tile=256, tiles=1024, grid=256,
                                           group_m=8, xcd_remap=1, **one)
    # 16384^3 bf16: 1 GiB of operands; 8 MiB A panels, 16 of them fit 128 MiB
    one["units"] = 4096
    assert P(bf, 16384, 16384, 16384) == dict(variant=18, tile=256, tiles=4096, grid=256,
                                              group_m=16, xcd_remap=2, **one)
    # fp8: 4 MiB panels, 32 rows per band
    assert P(f8, 16384, 16384, 16384) == dict(variant=0, tile=256, tiles=4096, grid=256,
                                              group_m=32, xcd_remap=2, **one)
    assert P(f8, 8192, 8192, 8192)["group_m"] == 8
    # exactly at the cache size (bf16 8192^3: 256 MiB) is not beyond it
    assert P(bf, 8192, 8192, 8192)["variant"] == 0
    # 8192 x 4096 x 14336: 336 MiB, 7 MiB panels -> 16 rows
    p = P(bf, 8192, 4096, 14336)
    assert (p["variant"], p["group_m"], p["xcd_remap"]) == (18, 16, 2)
    # fewer 256 x 256 tiles than compute units: 128 x 128 tiles, 2 per CU
    p = P(bf, 8192, 1024, 8192)
    assert (p["variant"], p["tile"], p["tiles"], p["grid"]) == (4, 128, 512, 512)
    p = P(bf, 8192, 1024, 8192, cus=64)          # a smaller device: 256-tiles fill it
    assert (p["variant"], p["tile"], p["grid"]) == (0, 256, 64)
    # explicit options are kept: band height, remap off, a chosen variant
    assert P(bf, 16384, 16384, 16384, group_m=8)[("group_m")] == 8
    assert P(bf, 16384, 16384, 16384, group_m=8)["xcd_remap"] == 1
    p = P(bf, 16384, 16384, 16384, xcd_remap=0)
    assert (p["group_m"], p["xcd_remap"]) == (16, 0)
    assert P(bf, 16384, 16384, 16384, variant=3)["variant"] == 3
    assert P(bf, 4096, 4096, 4096, xcd_remap=2)["xcd_remap"] == 2
    # grid option, band height clipped to the tile rows
    assert P(bf, 4096, 4096, 4096, grid=64)["grid"] == 64
    assert P(bf, 512, 65536, 64)["group_m"] == 2     # 2 x 256 tiles: 256-tiles
    assert P(bf, 512, 8192, 64)["group_m"] == 4      # 128-tiles: 4 tile rows
    # the 4-bit and MX products keep the grouped order at every size
    p = P(tkg.DTYPE_FP4_BLOCKSCALED, 16384, 16384, 16384)
    assert (p["group_m"], p["xcd_remap"]) == (8, 1)
    assert P(tkg.DTYPE_MXFP8, 16384, 16384, 16384)["xcd_remap"] == 1
    # empty products launch nothing; bad shapes and devices are rejected
    assert P(bf, 0, 64, 64)["grid"] == 0 and P(bf, 64, 64, 0)["grid"] > 0
    for args, kw in [((bf, 64, 64, 12), {}), ((f8, 64, 64, 8), {}),
                     ((bf, 64, 64, 64), {"cus": 0}), ((bf, 64, 64, 64), {"variant": 99}),
                     ((tkg.DTYPE_MXFP4, 64, 64, 64), {}), ((9, 64, 64, 64), {})]:
        with pytest.raises(tkg.TkgError):
            P(*args, **kw)


def test_plan_launch_tail_quadrants():
    # a partial last round of 256 x 256 tiles whose 128 x 128 quadrants fit
    # one round of the small-tile slots (2 per CU) runs as a second launch
    P = tkg.plan_launch
    bf, f8 = tkg.DTYPE_BF16, tkg.DTYPE_FP8
    p = P(bf, 6144, 6144, 6144)                 # 576 tiles: 2 rounds + 64
    assert (p["units"], p["tail_variant"], p["tail_units"], p["tail_grid"]) == (512, 4, 256, 256)
    p = P(f8, 4352, 4096, 1024)                 # 272 tiles: 1 round + 16
    assert (p["units"], p["tail_units"], p["tail_grid"]) == (256, 64, 64)
    p = P(bf, 6400, 6144, 512)                  # 600 tiles: 88 left, 352 <= 512
    assert (p["units"], p["tail_units"]) == (512, 352)
    # 400 tiles: 144 left, 576 quadrants > 512 slots: one launch
    assert P(bf, 5120, 5120, 4096)["tail_units"] == 0
    # 8448^2 x 8192 bf16: beyond the cache (5-slot ring, 32-row bands) and a tail
    p = P(bf, 8448, 8448, 8192)
    assert (p["variant"], p["group_m"], p["units"], p["tail_units"]) == (18, 32, 1024, 260)
    # whole rounds, ragged tiles, explicit grid or variant, K = 0: one launch
    for args, kw in [((bf, 8192, 8192, 8192), {}), ((bf, 6144, 6100, 1024), {}),
                     ((bf, 6144, 6144, 1024), {"grid": 256}),
                     ((bf, 6144, 6144, 1024), {"variant": 17}), ((bf, 6144, 6144, 0), {})]:
        p = P(*args, **kw)
        assert p["tail_units"] == 0 and p["tail_variant"] == -1 and p["units"] == p["tiles"], (args, kw)
    # fewer tiles than CUs: the small-tile configuration, one launch
    assert P(bf, 2048, 2048, 2048)["tail_units"] == 0
    # a smaller device: 576 tiles on 128 CUs leave 64, whose 256 quadrants
    # fill its 256 slots
    p = P(bf, 6144, 6144, 1024, cus=128)
    assert (p["grid"], p["units"], p["tail_units"], p["tail_grid"]) == (128, 512, 256, 256)


def test_device_info_without_or_with_a_device():
    # null outputs are rejected; without a usable device the call reports
    # TKG_ERR_DEVICE (it only queries the runtime)
    cus, clk = ctypes.c_int32(), ctypes.c_int32()
    assert L.tkg_device_info(None, ctypes.byref(clk)) == S["TKG_ERR_NULL"]
    assert L.tkg_device_info(ctypes.byref(cus), None) == S["TKG_ERR_NULL"]
    st = L.tkg_device_info(ctypes.byref(cus), ctypes.byref(clk))
    assert st in (S["TKG_OK"], S["TKG_ERR_DEVICE"])
    if st == S["TKG_OK"]:
        assert cus.value > 0 and clk.value > 0
