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

``cpu_baseline``: the CPU oracle (its decode of each format and its plain
fp64 C product, OpenMP) timed on a bounded sample of the same three
products, 64 x 64 output tiles of each in turn, for a context number; it is
test infrastructure and takes no part in the GPU path.

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


# sources only the attention kernel is built from
ATTN_SOURCES = ("attn_fwd.hip", "tkg_attn_layout.hpp")


def _code_only(text: str) -> str:
    """C++ source without its comments and whitespace (string and character
    literals kept), so that a comment edit leaves the hash of the code that
    was measured unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def kernel_source_hash(family: str = "gemm", read=None) -> str:
    """Hash of the code (comments and whitespace removed) of the kernel
    sources a family is built from (the GEMM family: every source but the
    attention-only files; attention: every source but the GEMM kernels).
    `read(name)` returns a source's text (default: the file in csrc/)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tiled_dense_gemm_amd", "csrc")
    if read is None:
        def read(name):
            return open(os.path.join(csrc, name), encoding="utf-8").read()
        names = os.listdir(csrc)
    else:
        names = read(None)
    for name in sorted(names):
        if not name.endswith((".hip", ".hpp")):
            continue
        if family == "gemm" and name in ATTN_SOURCES:
            continue
        if family == "attention" and name.startswith("gemm_"):
            continue
        h.update(name.encode())
        h.update(_code_only(read(name)).encode())
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


ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic.json")


def measured_attention_traffic(name: str):
    """HBM bytes per launch of an attention workload from the committed
    counter runs, or None when they were taken on other kernel sources."""
    try:
        rec = json.load(open(ATTN_TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash("attention"):
        return None
    k = rec.get("workloads", {}).get(name)
    return None if k is None else k.get("hbm_bytes_per_launch")


KERNEL_KEYS = {"gemm_dense_kernel<0": "gemm_bf16", "gemm_dense_kernel<1": "gemm_fp8",
               "gemm_fp4_kernel": "gemm_fp4_blockscaled", "gemm_mx_kernel<0": "gemm_mxfp4",
               "gemm_mx_kernel<1": "gemm_mxfp8"}
# MX products (e2m1 / e4m3 values with an E8M0 scale per 32) run on the
# scaled MFMAs at the 4-bit and 8-bit rates
PEAK_MX_TFLOPS = {"mxfp4": 10100.0, "mxfp8": 5000.0}


def _kernel_key(name: str):
    for frag, key in KERNEL_KEYS.items():
        if frag in name:
            return key
    return None


def _bench_line(path):
    """The JSON line a bench run printed (None without a log)."""
    if not path or not os.path.exists(path):
        return None
    line = None
    for l in open(path):
        if l.startswith("{") and '"metric"' in l:
            line = l
    return json.loads(line) if line else None


def summarize_profile(trace_dir: str, fetch_dir: str, write_dir: str,
                      size: int, out_md: str, out_json: str, command: str,
                      bench_log: str = None) -> int:
    """Turn rocprofv3 CSV output into the committed summaries.

    trace_dir: --kernel-trace --stats run of the timed bench;
    fetch_dir / write_dir: --pmc FETCH_SIZE / WRITE_SIZE runs of
    `bench.py --profile` (which ends with three 1 GiB device copies that
    calibrate the counters: bytes = counter * (1 GiB / counter_of_copy))."""
    import csv
    import glob
    import statistics

    def rows(d, pattern):
        out = []
        for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    # launches in start order; the summary keeps the last `steps` of each
    # kernel, the launches the bench run timed with HIP events (the others
    # are its warmup)
    bench = _bench_line(bench_log)
    steps = bench["steps"] if bench else None
    launches = {}
    for r in rows(trace_dir, "*kernel_trace.csv"):
        k = _kernel_key(r["Kernel_Name"])
        if k:
            launches.setdefault(k, []).append(
                (int(r["Start_Timestamp"]),
                 (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
    dur = {k: [d for _, d in sorted(v)][-steps:] if steps else [d for _, d in sorted(v)]
           for k, v in launches.items()}
    event_us = {}
    if bench:
        for k, v in list(bench.get("kernels", {}).items()) + list(
                (bench.get("next_rows") or {}).items()):
            if "ms_mean" in v:
                event_us[k] = v["ms_mean"] * 1e3

    def counter(d, cname):
        per, cal = {}, []
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            v = float(r["Counter_Value"])
            k = _kernel_key(r["Kernel_Name"])
            if k:
                per.setdefault(k, []).append(v)
            elif "copy" in r["Kernel_Name"] and v > 512 * 1024:
                cal.append(v)
        return per, cal

    fetch, fcal = counter(fetch_dir, "FETCH_SIZE")
    write, wcal = counter(write_dir, "WRITE_SIZE")
    gib_kib = 1024.0 * 1024.0
    ff = gib_kib / statistics.mean(fcal) if fcal else None
    fw = gib_kib / statistics.mean(wcal) if wcal else None
    M = N = K = size
    flops = 2.0 * M * N * K
    algo = {"gemm_bf16": (2 * M * K + 2 * N * K + 2 * M * N),
            "gemm_fp8": (M * K + N * K + 2 * M * N),
            "gemm_fp4_blockscaled": (M * K // 2 + N * K // 2 + M * K // 16
                                     + N * K // 16 + 2 * M * N),
            "gemm_mxfp4": (M * K // 2 + N * K // 2 + M * K // 32 + N * K // 32 + 2 * M * N),
            "gemm_mxfp8": (M * K + N * K + M * K // 32 + N * K // 32 + 2 * M * N)}
    rec = {"kernel_source_hash": kernel_source_hash(), "size": size,
           "copy_calibration": {"fetch_factor": ff, "write_factor": fw,
                                "copy_bytes": 1 << 30},
           "command": command, "kernels": {}}
    lines = ["# GEMM kernels at M=N=K=%d on one MI355X (rocprofv3)" % size, "",
             "Produced by:", "", "```", command, "```", "",
             ("Durations: the kernel trace's last %d launches of each kernel, the "
              "ones the traced bench run timed; beside them the mean that run's "
              "HIP events measured around the same launches." % steps) if steps else
             "Durations: every traced launch.", "",
             "| kernel | launches | mean us | min us | HIP-event mean us (same run) | TFLOP/s (mean) | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (calibrated) | compulsory bytes | ratio |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in ("gemm_bf16", "gemm_fp8", "gemm_fp4_blockscaled", "gemm_mxfp4", "gemm_mxfp8"):
        d = dur.get(k, [])
        if not d and k.startswith("gemm_mx"):
            continue
        fk = statistics.mean(fetch[k]) if fetch.get(k) else None
        wk = statistics.mean(write[k]) if write.get(k) else None
        hbm = (fk * 1024 * ff + wk * 1024 * fw) if (fk and wk and ff and fw) else None
        mean_us = statistics.mean(d) if d else None
        rec["kernels"][k] = {"launches": len(d), "mean_us": mean_us,
                             "min_us": min(d) if d else None,
                             "event_mean_us": event_us.get(k),
                             "fetch_kib": fk, "write_kib": wk,
                             "hbm_bytes_per_launch": hbm,
                             "compulsory_bytes": algo[k]}
        lines.append("| %s | %d | %s | %s | %s | %s | %s | %s | %s | %d | %s |" % (
            k, len(d), "%.1f" % mean_us if d else "-",
            "%.1f" % min(d) if d else "-",
            "%.1f" % event_us[k] if k in event_us else "-",
            "%.1f" % (flops / (mean_us * 1e-6) / 1e12) if d else "-",
            "%.0f" % fk if fk else "-", "%.0f" % wk if wk else "-",
            "%.3g" % hbm if hbm else "-", algo[k],
            "%.2f" % (hbm / algo[k]) if hbm else "-"))
    lines += ["", "Copy calibration: FETCH_SIZE factor %s, WRITE_SIZE factor %s "
              "(1 GiB copy / counter reading)." % (
                  "%.4f" % ff if ff else "-", "%.4f" % fw if fw else "-"), ""]
    # optional SQ/TCC counter passes: every other counter_collection.csv
    # under the trace dir's parent that is not the FETCH/WRITE pass
    extra = {}
    parent = os.path.dirname(os.path.abspath(trace_dir))
    for d in sorted(glob.glob(os.path.join(parent, "*"))):
        if os.path.abspath(d) in (os.path.abspath(fetch_dir), os.path.abspath(write_dir)):
            continue
        for r in rows(d, "*counter_collection.csv"):
            k = _kernel_key(r["Kernel_Name"])
            if k:
                extra.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    if extra:
        names = sorted({c for k in extra for c in extra[k]})
        lines += ["Other counters (mean per launch, summed over the device):", "",
                  "| counter | " + " | ".join(sorted(extra)) + " |",
                  "|---" * (len(extra) + 1) + "|"]
        for c in names:
            lines.append("| %s | " % c + " | ".join(
                "%.4g" % statistics.mean(extra[k][c]) if c in extra[k] else "-"
                for k in sorted(extra)) + " |")
        for k in sorted(extra):
            e = extra[k]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in e and "GRBM_GUI_ACTIVE" in e:
                # MFMA busy cycles per SIMD over GPU-active cycles per XCD
                util = (statistics.mean(e["SQ_VALU_MFMA_BUSY_CYCLES"]) / 1024.0) / (
                    statistics.mean(e["GRBM_GUI_ACTIVE"]) / 8.0)
                rec["kernels"][k]["mfma_busy_fraction"] = util
                lines.append("")
                lines.append("%s: MFMA busy %.1f%% of active cycles (1024 SIMDs, 8 XCDs)" % (k, 100 * util))
            if "SQ_LDS_BANK_CONFLICT" in e and "SQ_LDS_IDX_ACTIVE" in e:
                rec["kernels"][k]["lds_bank_conflict_over_active"] = (
                    statistics.mean(e["SQ_LDS_BANK_CONFLICT"]) /
                    max(1.0, statistics.mean(e["SQ_LDS_IDX_ACTIVE"])))
            if "TCC_HIT_sum" in e and "TCC_MISS_sum" in e:
                h, m = statistics.mean(e["TCC_HIT_sum"]), statistics.mean(e["TCC_MISS_sum"])
                rec["kernels"][k]["l2_hit_rate"] = h / (h + m)
        lines.append("")
    open(out_md, "w").write("\n".join(lines))
    json.dump(rec, open(out_json, "w"), indent=1)
    print("\n".join(lines))
    return 0


def _attention_workload(kname: str, grid_x: int, wg_x: int):
    """The ATTN_WORKLOADS entry a traced attention dispatch ran, from its
    kernel instance (head dimension, causal) and grid size."""
    import re
    m = re.search(r"attn_fwd_kernel<(\d+), (true|false)", kname)
    if not m or wg_x <= 0:
        return None
    D, causal = int(m.group(1)), m.group(2) == "true"
    bq = 32 * (wg_x // 64)
    for name, B, Hq, Hkv, N, d, c in ATTN_WORKLOADS:
        if d == D and c == causal and B * Hq * ((N + bq - 1) // bq) * wg_x == grid_x:
            return name
    return None


def summarize_attention_profile(trace_dir, fetch_dir, write_dir, out_md, out_json, command,
                                bench_log=None):
    """Committed summary of the attention kernels: durations from the
    --kernel-trace run of `bench.py --with-attn`, HBM bytes from the
    FETCH_SIZE / WRITE_SIZE runs of `bench.py --profile --with-attn`
    (calibrated by the 1 GiB copies at its end), other counter passes from
    sibling directories."""
    import csv
    import glob
    import statistics

    def rows(d, pattern):
        out = []
        for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    def key(r):
        gx = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        wx = int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size") or 0)
        return _attention_workload(r["Kernel_Name"], gx, wx)

    # as for the GEMMs: the last `steps` launches of each workload are the
    # ones the traced bench run timed with HIP events
    bench = _bench_line(bench_log)
    steps = bench["steps"] if bench else None
    launches = {}
    for r in rows(trace_dir, "*kernel_trace.csv"):
        k = key(r)
        if k:
            launches.setdefault(k, []).append(
                (int(r["Start_Timestamp"]),
                 (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
    dur = {k: [d for _, d in sorted(v)][-steps:] if steps else [d for _, d in sorted(v)]
           for k, v in launches.items()}
    event_us = {k: v["ms_mean"] * 1e3 for k, v in ((bench or {}).get("next_rows") or {}).items()
                if "ms_mean" in v}

    def counter(d, cname):
        per, cal = {}, []
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != cname:
                continue
            v = float(r["Counter_Value"])
            k = key(r) if "attn_fwd" in r["Kernel_Name"] else None
            if k:
                per.setdefault(k, []).append(v)
            elif "copy" in r["Kernel_Name"] and v > 512 * 1024:
                cal.append(v)
        return per, cal

    fetch, fcal = counter(fetch_dir, "FETCH_SIZE")
    write, wcal = counter(write_dir, "WRITE_SIZE")
    gib_kib = 1024.0 * 1024.0
    ff = gib_kib / statistics.mean(fcal) if fcal else None
    fw = gib_kib / statistics.mean(wcal) if wcal else None
    rec = {"kernel_source_hash": kernel_source_hash("attention"),
           "copy_calibration": {"fetch_factor": ff, "write_factor": fw, "copy_bytes": 1 << 30},
           "command": command, "workloads": {}}
    lines = ["# Attention forward kernels on one MI355X (rocprofv3)", "",
             "Produced by:", "", "```", command, "```", "",
             "Algorithmic flops: 4 D per visible (query, key) pair (Q K^T and P V); "
             "compulsory bytes: Q, K, V read once and O written once (bf16).", "",
             ("Durations: the kernel trace's last %d launches of each workload, the "
              "ones the traced bench run timed; beside them the mean that run's "
              "HIP events measured." % steps) if steps else "Durations: every traced launch.",
             "",
             "| workload | launches | mean us | min us | HIP-event mean us (same run) | TFLOP/s (mean) | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (calibrated) | compulsory bytes | ratio |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, B, Hq, Hkv, N, D, causal in ATTN_WORKLOADS:
        d = dur.get(name, [])
        fk = statistics.mean(fetch[name]) if fetch.get(name) else None
        wk = statistics.mean(write[name]) if write.get(name) else None
        hbm = (fk * 1024 * ff + wk * 1024 * fw) if (fk and wk and ff and fw) else None
        algo = 2 * D * (2 * B * Hq * N + 2 * B * Hkv * N)
        flops = attention_flops(B, Hq, N, D, causal)
        mean_us = statistics.mean(d) if d else None
        rec["workloads"][name] = {"launches": len(d), "mean_us": mean_us,
                                  "min_us": min(d) if d else None,
                                  "event_mean_us": event_us.get(name),
                                  "tflops": flops / (mean_us * 1e-6) / 1e12 if d else None,
                                  "fetch_kib": fk, "write_kib": wk,
                                  "hbm_bytes_per_launch": hbm, "compulsory_bytes": algo}
        lines.append("| %s | %d | %s | %s | %s | %s | %s | %s | %s | %d | %s |" % (
            name, len(d), "%.1f" % mean_us if d else "-", "%.1f" % min(d) if d else "-",
            "%.1f" % event_us[name] if name in event_us else "-",
            "%.1f" % (flops / (mean_us * 1e-6) / 1e12) if d else "-",
            "%.0f" % fk if fk else "-", "%.0f" % wk if wk else "-",
            "%.3g" % hbm if hbm else "-", algo, "%.2f" % (hbm / algo) if hbm else "-"))
    lines += ["", "Copy calibration: FETCH_SIZE factor %s, WRITE_SIZE factor %s." % (
        "%.4f" % ff if ff else "-", "%.4f" % fw if fw else "-"), ""]
    extra = {}
    parent = os.path.dirname(os.path.abspath(trace_dir))
    for dd in sorted(glob.glob(os.path.join(parent, "*"))):
        if os.path.abspath(dd) in (os.path.abspath(fetch_dir), os.path.abspath(write_dir)):
            continue
        for r in rows(dd, "*counter_collection.csv"):
            k = key(r) if "attn_fwd" in r["Kernel_Name"] else None
            if k:
                extra.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    if extra:
        names = sorted({c for k in extra for c in extra[k]})
        ks = [w[0] for w in ATTN_WORKLOADS if w[0] in extra]
        lines += ["Other counters (mean per launch, summed over the device):", "",
                  "| counter | " + " | ".join(ks) + " |", "|---" * (len(ks) + 1) + "|"]
        for c in names:
            lines.append("| %s | " % c + " | ".join(
                "%.4g" % statistics.mean(extra[k][c]) if c in extra[k] else "-" for k in ks) + " |")
        lines.append("")
        for k in ks:
            e = extra[k]
            if "SQ_LDS_BANK_CONFLICT" in e and "SQ_LDS_IDX_ACTIVE" in e:
                rec["workloads"][k]["lds_bank_conflict_over_active"] = (
                    statistics.mean(e["SQ_LDS_BANK_CONFLICT"]) /
                    max(1.0, statistics.mean(e["SQ_LDS_IDX_ACTIVE"])))
            if "GRBM_GUI_ACTIVE" in e and rec["workloads"][k]["mean_us"]:
                # GPU-active cycles per XCD over the launch: the average clock
                ghz = statistics.mean(e["GRBM_GUI_ACTIVE"]) / 8.0 / (rec["workloads"][k]["mean_us"] * 1e3)
                rec["workloads"][k]["clock_ghz_estimate"] = ghz
                lines.append("%s: about %.2f GHz over the launch (GRBM_GUI_ACTIVE per XCD / "
                             "traced duration)" % (k, ghz))
        lines.append("")
    open(out_md, "w").write("\n".join(lines))
    json.dump(rec, open(out_json, "w"), indent=1)
    print("\n".join(lines))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--size", type=int, default=8192)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--summarize-profile", nargs=3,
                    metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--profile-command", default="")
    ap.add_argument("--bench-log", default=None,
                    help="log of the traced bench run (its JSON line gives the timed "
                         "launch count and the HIP-event means)")
    ap.add_argument("--summarize-attn-profile", nargs=3,
                    metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--with-attn", action="store_true",
                    help="also time attention forward (tkg_attention_fwd) on its "
                         "workloads, reported under next_rows, outside the step "
                         "(the default; kept for older command lines)")
    ap.add_argument("--with-mx", action="store_true",
                    help="also time the MX products (gemm_mxfp4, gemm_mxfp8) on the "
                         "same shape, reported under next_rows, outside the step "
                         "(the default; kept for older command lines)")
    ap.add_argument("--no-attn", action="store_true", help="skip the attention rows")
    ap.add_argument("--no-mx", action="store_true", help="skip the MX rows")
    args = ap.parse_args()
    args.with_attn = not args.no_attn
    args.with_mx = not args.no_mx

    if args.summarize_profile:
        return summarize_profile(
            *args.summarize_profile, args.size,
            os.path.join(ROOT, "profiles", "gemm_kernels_%d.md" % args.size),
            TRAFFIC_FILE if args.size == 8192 else
            os.path.join(ROOT, "profiles", "traffic_%d.json" % args.size),
            args.profile_command, args.bench_log)

    if args.summarize_attn_profile:
        return summarize_attention_profile(
            *args.summarize_attn_profile,
            os.path.join(ROOT, "profiles", "attention_fwd.md"), ATTN_TRAFFIC_FILE,
            args.profile_command, args.bench_log)

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
    extra = {}
    if args.with_mx:
        Am4, Asm4 = gdev.mx_operand(6, M, K, "e2m1", device=dev)
        Bm4, Bsm4 = gdev.mx_operand(7, N, K, "e2m1", device=dev)
        Am8, Asm8 = gdev.mx_operand(8, M, K, "e4m3", device=dev)
        Bm8, Bsm8 = gdev.mx_operand(9, N, K, "e4m3", device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    calls = {
        "bf16": lambda: tkg.gemm_bf16(A16, B16, out=C, stream=stream),
        "fp8": lambda: tkg.gemm_fp8(A8, sa, B8, sb, out=C, stream=stream),
        "fp4_blockscaled": lambda: tkg.gemm_fp4_blockscaled(
            A4, As4, ta, B4, Bs4, tb, out=C, stream=stream),
    }
    names = list(calls)
    if args.with_mx:
        extra = {
            "mxfp4": lambda: tkg.gemm_mxfp4(Am4, Asm4, Bm4, Bsm4, out=C, stream=stream),
            "mxfp8": lambda: tkg.gemm_mxfp8(Am8, Asm8, Bm8, Bsm8, out=C, stream=stream),
        }

    for _ in range(args.warmup):
        for k in names:
            calls[k]()
    torch.cuda.synchronize()

    if args.profile:
        for _ in range(args.steps):
            for k in names:
                calls[k]()
        for _ in range(args.steps):
            for k in extra:
                extra[k]()
        torch.cuda.synchronize()
        if args.with_attn:
            profile_attention(args, dev, stream)
        # calibration copy: 1 GiB read + 1 GiB written
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
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

    # the MX products, timed apart from the step (not part of `value`)
    next_rows = None
    if extra:
        next_rows = {}
        for k, fn in extra.items():
            for _ in range(args.warmup):
                fn()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            torch.cuda.synchronize()
            for e0, e1 in evs:
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            t = [e0.elapsed_time(e1) for e0, e1 in evs]
            ms = float(np.mean(t))
            tf = flops / (ms * 1e-3) / 1e12
            next_rows["gemm_" + k] = {
                "ms_mean": round(ms, 4), "ms_min": round(float(np.min(t)), 4),
                "tflops": round(tf, 1), "peak_tflops": PEAK_MX_TFLOPS[k],
                "frac_of_peak": round(tf / PEAK_MX_TFLOPS[k], 4)}

    if args.with_attn:
        next_rows = next_rows or {}
        next_rows.update(time_attention(args, dev, stream))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(((A16, B16), (A8, sa, B8, sb), (A4, As4, ta, B4, Bs4, tb)),
                           args.cpu_seconds)

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
    if next_rows is not None:
        out["next_rows"] = next_rows
    print(json.dumps(out), flush=True)
    return 0


# attention forward workloads: (name, B, Hq, Hkv, N, D, causal). The pages
# fix head dimension 64 / 128, sequence lengths 1024..16384, causal,
# non-causal and grouped-query; batch and heads are this benchmark's choice
# (model width 2048 = Hq * D).
ATTN_WORKLOADS = [
    ("attn_fwd_d128", 16, 16, 16, 4096, 128, False),
    ("attn_fwd_d128_causal", 16, 16, 16, 4096, 128, True),
    ("attn_fwd_d64", 16, 32, 32, 4096, 64, False),
    ("attn_fwd_d128_gqa8_causal_n16k", 1, 16, 2, 16384, 128, True),
]


def attention_flops(B, Hq, N, D, causal):
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4.0 * D * B * Hq * pairs


def _attention_inputs(dev, B, Hq, Hkv, N, D):
    import torch

    import gemm_inputs.device as gdev
    Q = gdev.bf16_operand(20, B * Hq * N, D, device=dev).view(B, Hq, N, D)
    K = gdev.bf16_operand(21, B * Hkv * N, D, device=dev).view(B, Hkv, N, D)
    V = gdev.bf16_operand(22, B * Hkv * N, D, device=dev).view(B, Hkv, N, D)
    return Q, K, V, torch.empty_like(Q)


def profile_attention(args, dev, stream):
    """`steps` untimed launches of each attention workload (profiler runs)."""
    import torch

    import tiled_dense_gemm_amd as tkg
    for name, B, Hq, Hkv, N, D, causal in ATTN_WORKLOADS:
        Q, K, V, O = _attention_inputs(dev, B, Hq, Hkv, N, D)
        for _ in range(args.steps):
            tkg.tkg_attention_fwd(Q, K, V, causal=causal, out=O, stream=stream)
        torch.cuda.synchronize()
        del Q, K, V, O
        torch.cuda.empty_cache()


def time_attention(args, dev, stream):
    import numpy as np
    import torch

    import tiled_dense_gemm_amd as tkg

    rows = {}
    for name, B, Hq, Hkv, N, D, causal in ATTN_WORKLOADS:
        Q, K, V, O = _attention_inputs(dev, B, Hq, Hkv, N, D)
        fn = lambda: tkg.tkg_attention_fwd(Q, K, V, causal=causal, out=O, stream=stream)
        for _ in range(args.warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        t = [e0.elapsed_time(e1) for e0, e1 in evs]
        ms = float(np.mean(t))
        tf = attention_flops(B, Hq, N, D, causal) / (ms * 1e-3) / 1e12
        rows[name] = {
            "workload": "B=%d Hq=%d Hkv=%d N=%d D=%d %s, bf16 N(0,1) inputs"
                        % (B, Hq, Hkv, N, D, "causal" if causal else "non-causal"),
            "ms_mean": round(ms, 4), "ms_min": round(float(np.min(t)), 4),
            "tflops": round(tf, 1), "peak_tflops": PEAK_TFLOPS["bf16"],
            "frac_of_peak": round(tf / PEAK_TFLOPS["bf16"], 4),
            "hbm_bytes_per_launch": measured_attention_traffic(name)}
        del Q, K, V, O
        torch.cuda.empty_cache()
    return rows


def cpu_baseline(ops, seconds):
    """The oracle on 64x64 output tiles of the step's three products (bf16,
    fp8, block-scaled 4-bit, in turn: the oracle's own decode and fp64
    product for each format) until `seconds` of CPU time are spent; the
    rate is the tiles' FLOP over that time, in TFLOP/s."""
    import numpy as np
    import torch

    import oracle

    def rows(x, r0):
        t = x[r0:r0 + 64]
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    (A16, B16), (A8, sa, B8, sb), (A4, As4, ta, B4, Bs4, tb) = ops
    K = A16.shape[1]
    M, N = A16.shape[0], B16.shape[0]
    rng = np.random.default_rng(0)
    done = [0, 0, 0]
    t_used = 0.0
    while t_used < seconds or min(done) < 2:
        f = (done[0] + done[1] + done[2]) % 3
        i0 = int(rng.integers(0, M - 64 + 1))
        j0 = int(rng.integers(0, N - 64 + 1))
        if f == 0:
            args = (rows(A16, i0), rows(B16, j0))
            fn = oracle.gemm_bf16
        elif f == 1:
            args = (rows(A8, i0), sa, rows(B8, j0), sb)
            fn = oracle.gemm_fp8
        else:
            args = (rows(A4, i0), rows(As4, i0), ta, rows(B4, j0), rows(Bs4, j0), tb)
            fn = oracle.gemm_fp4_blockscaled
        t = time.perf_counter()
        fn(*args)
        t_used += time.perf_counter() - t
        done[f] += 1
    rate = sum(done) * 2.0 * 64 * 64 * K / t_used / 1e12
    return {"value": round(rate, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d random 64x64 output tiles each of the %d^3 bf16, fp8 and "
                      "block-scaled 4-bit products, in turn (the oracle's decode and "
                      "fp64 plain C product, %.1f s)" % (min(done), K, t_used)}


if __name__ == "__main__":
    sys.exit(main())
