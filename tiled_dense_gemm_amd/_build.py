"""Build step for the HIP library ``libtkg.so`` (gfx950).

``python tiled_dense_gemm_amd/_build.py`` compiles every ``csrc/*.hip`` file
for gfx950 with hipcc and links them into ``tiled_dense_gemm_amd/libtkg.so``
in place. The build is always done from scratch (seconds per file). The
script imports nothing from its package, so it runs before the library
exists (the package itself loads the library on import).
"""
from __future__ import annotations

import glob
import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtkg.so")
OBJDIR = os.path.join(PKG, "_build_obj")
# per-kernel register, scratch and LDS use as the compiler reports it
RESOURCES = os.path.join(OBJDIR, "kernel_resources.json")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + ["-Rpass-analysis=kernel-resource-usage",
                                             "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    lines = r.stdout.splitlines()
    res = [l for l in lines if "kernel-resource-usage" in l]
    out = "\n".join(l for l in lines if "is not a recognized feature" not in l
                    and "kernel-resource-usage" not in l and not l.startswith("  ")
                    and l.strip() not in ("^", "|"))
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(lines)))
    if out.strip() and verbose:
        print(out, flush=True)
    return obj, res


def _parse_resources(remarks):
    """{kernel symbol: {field: value}} from the compiler's
    kernel-resource-usage remarks."""
    kernels, cur = {}, None
    for l in remarks:
        m = re.search(r"remark:\s+Function Name: (\S+)", l)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", l)
        if m and cur is not None:
            v = m.group(2)
            cur[m.group(1).strip()] = int(v) if v.lstrip("-").isdigit() else v
    return kernels


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(lambda s: _compile(s, verbose), srcs))
    objs = [o for o, _ in done]
    resources = {}
    for _, rem in done:
        resources.update(_parse_resources(rem))
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + [
        "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    print("built", LIB)
