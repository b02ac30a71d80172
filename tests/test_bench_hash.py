"""bench.py keys its stored counter measurements (profiles/*traffic*.json) to
a hash of the kernel code with comments and whitespace removed: a comment
edit keeps the measurement, any code edit drops it."""
import bench


def test_code_only_strips_comments_and_keeps_literals():
    src = 'a = "x // y"; // note\n/* block\n comment */ b = \'/\';\nc = "q\\"/*";'
    assert bench._code_only(src) == 'a="x // y";b=\'/\';c="q\\"/*";'


def _hash_with(files, fam="gemm"):
    def read(name):
        return list(files) if name is None else files[name]
    return bench.kernel_source_hash(fam, read)


def test_hash_ignores_comments_not_code():
    base = {"gemm_dense.hip": "int f() { return 1; }  // one\n",
            "tkg_device.hpp": "/* helpers */\nint g();\n",
            "attn_fwd.hip": "int h();\n"}
    h0 = _hash_with(base)
    commented = dict(base, **{"gemm_dense.hip": "// header\nint f()  {\n  return 1;   // one!\n}\n"})
    assert _hash_with(commented) == h0
    changed = dict(base, **{"gemm_dense.hip": "int f() { return 2; }\n"})
    assert _hash_with(changed) != h0
    # the attention-only source is outside the GEMM family's hash
    assert _hash_with(dict(base, **{"attn_fwd.hip": "int h2();\n"})) == h0
    assert _hash_with(dict(base, **{"attn_fwd.hip": "int h2();\n"}), "attention") != \
        _hash_with(base, "attention")



def test_launch_log_attribution():
    # a traced run: per kernel family, launches in start order; the launch
    # log says which workload ran how many warmup and timed launches
    launches = {"gemm_bf16": [(t, float(t)) for t in range(1, 31)],
                "gemm_fp8": [(t, 100.0 + t) for t in range(5)],
                "gemm_mxfp4": [(t, 7.0) for t in range(3)]}
    blocks = [{"name": "step_bf16", "key": "gemm_bf16", "warmup": 5, "timed": 10},
              {"name": "step_fp8", "key": "gemm_fp8", "warmup": 2, "timed": 3},
              {"name": "bf16_4096", "key": "gemm_bf16", "warmup": 10, "timed": 5}]
    got = bench._attribute(launches, blocks)
    assert got["step_bf16"] == [float(t) for t in range(6, 16)]
    assert got["bf16_4096"] == [float(t) for t in range(26, 31)]
    assert got["step_fp8"] == [102.0, 103.0, 104.0]
    assert got["gemm_mxfp4"] == [7.0, 7.0, 7.0]   # not in the log: whole family
