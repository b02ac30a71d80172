"""Benchmark: GEMM TFLOP/s at M = N = K = 8192 on one MI355X.

One step is one pass of the whole hot path over synthetic operands already
resident in HBM: gemm_bf16, gemm_fp8 (per-tensor scales) and
gemm_fp4_blockscaled (e2m1 values, e4m3 block scales per 16, fp32 tensor
scales), each 8192 x 8192 x 8192 with bf16 output. ``value`` is the step's
counted flops (3 x 2 M N K) over its time; the per-kernel rates and their
fractions of the MI355X dense MFMA peak are in ``kernels``; ``roofline``
covers the kernel that takes the longest. Timing: W untimed warmup steps,
then K timed steps between synchronizations, with HIP events around every
launch on the stream the kernels run on (the pages time 10 warmup + 10
timed iterations, page "ThunderKittens: Simple, Fast, and Adorable AI
Kernels", section 5 "Evaluation Methodology").

``cpu_baseline``: the CPU oracle (plain fp64 C, OpenMP) timed on a bounded
sample of the same bf16 product, 64 x 64 output tiles, for a context
number; it is test infrastructure and takes no part in the GPU path.

``--profile`` runs only the GPU part (for rocprofv3) plus a 1 GiB device
copy that calibrates the HBM byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s at 8192^3 bf16 and fp8 on 1 MI355X; % of dense MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4_blockscaled": 2500.0}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_8192.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_dense_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter runs, or None when
    they were taken on other kernel sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--size", type=int, default=8192)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (a GEMM shards by splitting N across GPUs with no "
              "exchange; the per-GPU kernel is the one measured here).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gemm_inputs.device as gdev
    import tiled_dense_gemm_amd as tkg

    assert torch.cuda.is_available(), "bench.py needs the HIP device"
    dev = torch.device("cuda:0")
    n = args.size
    M = N = K = n
    flops = 2.0 * M * N * K

    # operands resident in HBM before timing
    A16 = gdev.bf16_operand(0, M, K, std=K ** -0.5, device=dev)
    B16 = gdev.bf16_operand(1, N, K, std=K ** -0.5, device=dev)
    A8, sa = gdev.fp8_operand(2, M, K, device=dev)
    B8, sb = gdev.fp8_operand(3, N, K, device=dev)
    A4, As4, ta = gdev.fp4_operand(4, M, K, device=dev)
    B4, Bs4, tb = gdev.fp4_operand(5, N, K, device=dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    calls = {
        "bf16": lambda: tkg.gemm_bf16(A16, B16, out=C, stream=stream),
        "fp8": lambda: tkg.gemm_fp8(A8, sa, B8, sb, out=C, stream=stream),
        "fp4_blockscaled": lambda: tkg.gemm_fp4_blockscaled(
            A4, As4, ta, B4, Bs4, tb, out=C, stream=stream),
    }
    names = list(calls)

    for _ in range(args.warmup):
        for k in names:
            calls[k]()
    torch.cuda.synchronize()

    if args.profile:
        for _ in range(args.steps):
            for k in names:
                calls[k]()
        torch.cuda.synchronize()
        # calibration copy: 1 GiB read + 1 GiB written
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("profile run done: %d steps of %s at %d^3; 3 copies of 1 GiB"
              % (args.steps, "+".join(names), n), flush=True)
        return 0

    # events on the stream the kernels are launched on
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, k in enumerate(names):
            calls[k]()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {k: [] for k in names}
    for s in range(args.steps):
        for i, k in enumerate(names):
            per[k].append(ev[s][i].elapsed_time(ev[s][i + 1]))
    step_ms = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(args.steps)) / args.steps
    kernels = {}
    for k in names:
        ms = float(np.mean(per[k]))
        tf = flops / (ms * 1e-3) / 1e12
        kernels["gemm_" + k] = {
            "ms_mean": round(ms, 4), "ms_min": round(float(np.min(per[k])), 4),
            "ms_median": round(float(np.median(per[k])), 4),
            "tflops": round(tf, 1), "peak_tflops": PEAK_TFLOPS[k],
            "frac_of_peak": round(tf / PEAK_TFLOPS[k], 4)}
    value = len(names) * flops / (step_ms * 1e-3) / 1e12

    dom = max(names, key=lambda k: kernels["gemm_" + k]["ms_mean"])
    dk = kernels["gemm_" + dom]
    roofline = {"bound": "mfma", "achieved": dk["tflops"],
                "peak": PEAK_TFLOPS[dom], "unit": "TFLOP/s",
                "frac": round(dk["tflops"] / PEAK_TFLOPS[dom], 4),
                "traffic": measured_traffic("gemm_" + dom),
                "kernel": "gemm_" + dom}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(A16, B16, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp8+fp4",
        "data": "synthetic",
        "config": {"workload": "C = A*B at M=N=K=%d: bf16 (A, B ~ N(0,1)/sqrt(K)), "
                               "fp8 e4m3 with per-tensor amax/448 scales, and "
                               "block-scaled e2m1 (e4m3 scale per 16, fp32 tensor "
                               "scale); A row-major, B column-major, bf16 C" % n,
                   "M": M, "N": N, "K": K, "global_batch": 1, "seq_len": None,
                   "parallelism": "single GPU"},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(A16, B16, seconds):
    """The oracle on 64x64 output tiles of the bf16 product until `seconds`
    of CPU time are spent; the rate is scaled to TFLOP/s."""
    import numpy as np
    import torch

    import oracle
    from oracle.formats import decode_bf16

    K = A16.shape[1]
    rng = np.random.default_rng(0)
    done = 0
    t_used = 0.0
    while t_used < seconds or done < 2:
        i0 = int(rng.integers(0, A16.shape[0] - 64 + 1))
        j0 = int(rng.integers(0, B16.shape[0] - 64 + 1))
        a = decode_bf16(A16[i0:i0 + 64].view(torch.int16).cpu().numpy().view(np.uint16))
        b = decode_bf16(B16[j0:j0 + 64].view(torch.int16).cpu().numpy().view(np.uint16))
        t = time.perf_counter()
        oracle.gemm_f64(a, b)
        t_used += time.perf_counter() - t
        done += 1
    rate = done * 2.0 * 64 * 64 * K / t_used / 1e12
    return {"value": round(rate, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d random 64x64 output tiles of the %d^3 bf16 product "
                      "(fp64 plain C oracle, %.1f s)" % (done, K, t_used)}


if __name__ == "__main__":
    sys.exit(main())
