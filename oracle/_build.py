"""Build step for the oracle's C reference GEMM (test infrastructure).

``python -m oracle._build`` compiles ``ref_gemm.c`` with gcc into
``oracle/libref_gemm.so``. The compile flags keep IEEE semantics (no
-ffast-math), so every output element is summed in the order written.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ref_gemm.c")
LIB = os.path.join(HERE, "libref_gemm.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
