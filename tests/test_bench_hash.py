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

