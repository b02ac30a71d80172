"""Benchmark: GEMM TFLOP/s at M = N = K = 8192 on one MI355X.

One step is one pass of the whole hot path over synthetic operands already
resident in HBM: gemm_bf16, gemm_fp8 (per-tensor scales) and
gemm_fp4_blockscaled (e2m1 values, e4m3 block scales per 16, fp32 tensor
scales), each 8192 x 8192 x 8192 with bf16 output. ``headline`` gives the
metric itself: bf16 and fp8 TFLOP/s and their fractions of the MI355X dense
MFMA peak. ``value`` is the step's counted flops (3 x 2 M N K) over its
time; ``kernels`` the per-product rates; ``rooflines`` one entry per
product (the 4-bit one against the fp16 rate it issues and against the fp4
dense peak), with HBM traffic, MFMA busy fraction and clock from the
committed counter runs of the same kernel code; ``roofline`` repeats the
entry of the step's longest kernel. Timing: W untimed warmup steps, then K
timed steps between synchronizations, with HIP events around every launch
on the stream the kernels run on (the pages time 10 warmup + 10 timed
iterations, page "ThunderKittens: Simple, Fast, and Adorable AI Kernels",
section 5 "Evaluation Methodology").

``configs``: every other configuration of the workload list (256^3 to
16384^3 and the FFN shapes in bf16, fp8 16384^3, the 4-bit product at
16384^3 and 65536^3, and one GPU's N/8 shard of 8192^3), each timed on its
own operands after the step. ``next_rows``: the MX products and attention
forward. ``launch_log``: every GEMM launch of the run in dispatch order, so
a kernel trace of the same run can be attributed launch by launch.

``cpu_baseline``: the CPU oracle (its decode of each format and its plain
fp64 C product, OpenMP) timed on a bounded sample of the same three
products -- full-width row panels -- for a context number, with the host's
CPU model and thread count; it is test infrastructure and takes no part in
the GPU path.

``--profile`` runs only the step's products (and the MX and attention
rows) for rocprofv3 counter passes, plus 1 GiB device copies that
calibrate the HBM byte counters.
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
# MI355X published dense MFMA peaks (TFLOP/s). The block-scaled 4-bit
# product (e4m3 scale per 16) runs exact fp16 MFMAs, so its row carries the
# fp16 rate it issues and, beside it, the fp4 dense peak.
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4_blockscaled": 2500.0}
PEAK_FP4_DENSE = 10100.0
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


def measured(kernel: str, field: str):
    """A per-kernel figure of the committed counter runs (traffic_8192.json),
    or None when they were taken on other kernel sources."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get(field)


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed counter runs, or None when
    they were taken on other kernel sources."""
    return measured(kernel, "hbm_bytes_per_launch")


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
SHADER_ENGINES = 32     # 8 XCDs x 4 shader engines (arrays) on MI355X


def _active_cycles(counters):
    """Active shader cycles of one launch, per shader engine (None when not
    collected). SQ_BUSY_CYCLES is summed over the chip's 32 shader engines
    (8 XCDs x 4; the profiler's agent record lists 32 arrays), so its mean
    per engine counts the cycles the kernel's waves occupied the arrays.
    GRBM_GUI_ACTIVE also counts front-end activity around the launch: in a
    counter run it has read up to 1.8x the shader engines' cycles for one
    launch, which would inflate a clock and deflate a busy fraction."""
    import statistics
    if counters.get("SQ_BUSY_CYCLES"):
        return statistics.mean(counters["SQ_BUSY_CYCLES"]) / SHADER_ENGINES
    return None


def _issue_mix(counters):
    """How a kernel's issue splits between the matrix cores and the other
    vector ALU work (None when not collected), per SIMD as fractions of the
    active cycles: MFMA busy; VALU busy (SQ_ACTIVE_INST_VALU, quad-cycles
    summed over the SIMD's waves, MFMA issue included); both at once
    (SQ_VALU_MFMA_COEXEC_CYCLES); and VALU instructions per MFMA
    (SQ_INSTS_VALU counts the MFMAs too) and exp2 (transcendental)
    instructions per MFMA."""
    import statistics
    act = _active_cycles(counters)
    need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES",
            "SQ_INSTS_VALU", "SQ_INSTS_MFMA")
    if not act or any(not counters.get(c) for c in need):
        return None
    m = lambda c: statistics.mean(counters[c])
    simds = 1024.0
    out = {"mfma_busy": m("SQ_VALU_MFMA_BUSY_CYCLES") / simds / act,
           "valu_busy": m("SQ_ACTIVE_INST_VALU") * 4 / simds / act,
           "valu_mfma_coexec": m("SQ_VALU_MFMA_COEXEC_CYCLES") / simds / act,
           "valu_per_mfma": m("SQ_INSTS_VALU") / m("SQ_INSTS_MFMA"),
           "trans_per_mfma": (m("SQ_INSTS_VALU_TRANS_F32") / m("SQ_INSTS_MFMA")
                              if counters.get("SQ_INSTS_VALU_TRANS_F32") else None)}
    text = ("MFMA busy %.2f, VALU busy %.2f (MFMA issue included), both at once %.2f of the "
            "active cycles; %.2f VALU instructions per MFMA (MFMAs counted)" % (
                out["mfma_busy"], out["valu_busy"], out["valu_mfma_coexec"], out["valu_per_mfma"]))
    if out["trans_per_mfma"] is not None:
        text += ", %.2f exp2 per MFMA" % out["trans_per_mfma"]
    return out, text


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


def _attribute(launches, blocks):
    """Split each kernel family's launches (in start order) over the bench
    run's launch log: {workload name: [durations of its timed launches]}.
    Families absent from the log are returned whole under their key."""
    out, pos = {}, {}
    for b in blocks:
        k = b["key"]
        seq = launches.get(k, [])
        i = pos.get(k, 0)
        out[b["name"]] = [d for _, d in seq[i + b["warmup"]:i + b["warmup"] + b["timed"]]]
        pos[k] = i + b["warmup"] + b["timed"]
    for k, seq in launches.items():
        if k not in pos:
            out[k] = [d for _, d in seq]
    return out


def summarize_profile(trace_dir: str, fetch_dir: str, write_dir: str,
                      size: int, out_md: str, out_json: str, command: str,
                      bench_log: str = None) -> int:
    """Turn rocprofv3 CSV output into the committed summaries.

    trace_dir: --kernel-trace --stats run of the timed bench, whose launch
    log (bench_log) attributes every traced launch to its workload;
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

    bench = _bench_line(bench_log)
    launches = {}
    for r in rows(trace_dir, "*kernel_trace.csv"):
        k = _kernel_key(r["Kernel_Name"])
        if k:
            launches.setdefault(k, []).append(
                (int(r["Start_Timestamp"]),
                 (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
    for k in launches:
        launches[k].sort()
    blocks = (bench or {}).get("launch_log") or []
    by_name = _attribute(launches, blocks)
    step_of = {"gemm_" + k: "step_" + k for k in ("bf16", "fp8", "fp4_blockscaled")}
    step_of.update({"gemm_mxfp4": "next_mxfp4", "gemm_mxfp8": "next_mxfp8"})
    dur = {k: by_name.get(step_of[k], by_name.get(k, [])) for k in step_of}
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
           "command": command, "kernels": {}, "configs": {}}
    lines = ["# GEMM kernels at M=N=K=%d on one MI355X (rocprofv3)" % size, "",
             "Produced by:", "", "```", command, "```", "",
             "Durations: the kernel trace's launches that the traced bench run timed "
             "with HIP events (its launch log names every launch's workload and "
             "warmup/timed role); beside them that run's HIP-event means.", "",
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
    cfg = (bench or {}).get("configs") or {}
    if cfg:
        lines += ["The other configurations, timed after the step in the same traced run:",
                  "", "| workload | dtype | M x N x K | launches | trace mean us | "
                  "HIP-event mean us | TFLOP/s (trace) | fraction of peak |",
                  "|---|---|---|---|---|---|---|---|"]
        for name, c in cfg.items():
            d = by_name.get(name, [])
            if not d:
                continue
            mean_us = statistics.mean(d)
            cf = 2.0 * c["M"] * c["N"] * c["K"]
            tf = cf / (mean_us * 1e-6) / 1e12
            frac = tf / c["peak_tflops"]
            rec["configs"][name] = {"launches": len(d), "mean_us": mean_us,
                                    "event_mean_us": c["ms_mean"] * 1e3, "tflops": tf,
                                    "frac_of_peak": frac}
            extra_frac = ""
            if c["dtype"] == "fp4_blockscaled":
                extra_frac = " (%.3f of the fp4 dense peak)" % (tf / PEAK_FP4_DENSE)
                rec["configs"][name]["frac_of_fp4_dense_peak"] = tf / PEAK_FP4_DENSE
            lines.append("| %s | %s | %dx%dx%d | %d | %.1f | %.1f | %.1f | %.3f%s |" % (
                name, c["dtype"], c["M"], c["N"], c["K"], len(d), mean_us,
                c["ms_mean"] * 1e3, tf, frac, extra_frac))
        lines.append("")
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
            if k not in rec["kernels"]:
                continue
            act = _active_cycles(e)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in e and act:
                # MFMA busy cycles per SIMD over active cycles per shader engine
                util = (statistics.mean(e["SQ_VALU_MFMA_BUSY_CYCLES"]) / 1024.0) / act
                rec["kernels"][k]["mfma_busy_fraction"] = util
                lines.append("")
                lines.append("%s: MFMA busy %.1f%% of active cycles (1024 SIMDs; SQ_BUSY_CYCLES "
                             "over %d shader engines)" % (k, 100 * util, SHADER_ENGINES))
            if act and rec["kernels"][k].get("mean_us"):
                # active cycles per shader engine over the traced launch
                # duration: the average shader clock of the launch
                ghz = act / (rec["kernels"][k]["mean_us"] * 1e3)
                rec["kernels"][k]["clock_ghz_estimate"] = ghz
                lines.append("%s: about %.2f GHz over the launch (SQ_BUSY_CYCLES per shader "
                             "engine / traced duration)" % (k, ghz))
            mix = _issue_mix(e)
            if mix:
                rec["kernels"][k]["issue_mix"] = mix[0]
                lines.append("%s: per SIMD, %s" % (k, mix[1]))
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
            act = _active_cycles(e)
            if act and rec["workloads"][k]["mean_us"]:
                # active cycles per shader engine over the launch: the average clock
                ghz = act / (rec["workloads"][k]["mean_us"] * 1e3)
                rec["workloads"][k]["clock_ghz_estimate"] = ghz
                lines.append("%s: about %.2f GHz over the launch (SQ_BUSY_CYCLES per shader "
                             "engine / traced duration)" % (k, ghz))
            mix = _issue_mix(e)
            if mix:
                rec["workloads"][k]["issue_mix"] = mix[0]
                lines.append("%s: per SIMD, %s" % (k, mix[1]))
        lines.append("")
    open(out_md, "w").write("\n".join(lines))
    json.dump(rec, open(out_json, "w"), indent=1)
    print("\n".join(lines))
    return 0


# Every BASELINE configuration beyond the step, timed after it: (name, dtype,
# M, N, K, operand std (None = 1/sqrt(K)), warmup, timed launches). The
# N/8 shard is one GPU's share of the 8192^3 product split over 8 GPUs.
CONFIGS = [
    ("bf16_256", "bf16", 256, 256, 256, 1.0, 10, 20),
    ("bf16_1024", "bf16", 1024, 1024, 1024, None, 10, 20),
    ("bf16_2048", "bf16", 2048, 2048, 2048, None, 10, 20),
    ("bf16_4096", "bf16", 4096, 4096, 4096, None, 10, 10),
    ("bf16_16384", "bf16", 16384, 16384, 16384, None, 3, 10),
    ("bf16_ffn_up_8192x14336x4096", "bf16", 8192, 14336, 4096, None, 5, 10),
    ("bf16_ffn_down_8192x4096x14336", "bf16", 8192, 4096, 14336, None, 5, 10),
    ("bf16_shard_8192x1024x8192", "bf16", 8192, 1024, 8192, None, 5, 10),
    ("fp8_16384", "fp8", 16384, 16384, 16384, 1.0, 3, 10),
    ("fp8_shard_8192x1024x8192", "fp8", 8192, 1024, 8192, 1.0, 5, 10),
    ("fp4_16384", "fp4_blockscaled", 16384, 16384, 16384, 1.0, 3, 10),
    ("fp4_65536", "fp4_blockscaled", 65536, 65536, 65536, 1.0, 1, 3),
]


class LaunchLog:
    """Times blocks of launches with HIP events on the launching stream and
    records, in dispatch order, which kernel family ran how many warmup and
    timed launches for which workload, so a kernel trace of the same run
    can be attributed launch by launch."""

    def __init__(self, stream):
        self.stream = stream
        self.blocks = []

    def time(self, name, key, fn, warmup, steps):
        import numpy as np
        import torch
        for _ in range(warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(self.stream)
        for i in range(steps):
            fn()
            ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        t = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        self.blocks.append({"name": name, "key": key, "warmup": warmup, "timed": steps})
        return {"ms_mean": round(float(np.mean(t)), 4), "ms_min": round(float(np.min(t)), 4),
                "ms_median": round(float(np.median(t)), 4)}


def _rate(flops, ms, peak):
    tf = flops / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 1), "peak_tflops": peak, "frac_of_peak": round(tf / peak, 4)}


def _operands(gdev, dtype, M, N, K, std, dev, seed):
    if dtype == "bf16":
        sd = K ** -0.5 if std is None else std
        return (gdev.bf16_operand(seed, M, K, std=sd, device=dev),
                gdev.bf16_operand(seed + 1, N, K, std=sd, device=dev))
    if dtype == "fp8":
        A, sa = gdev.fp8_operand(seed, M, K, device=dev)
        B, sb = gdev.fp8_operand(seed + 1, N, K, device=dev)
        return A, sa, B, sb
    A, As, ta = gdev.fp4_operand(seed, M, K, device=dev)
    B, Bs, tb = gdev.fp4_operand(seed + 1, N, K, device=dev)
    return A, As, ta, B, Bs, tb


def _call(tkg, dtype, ops, C, stream):
    if dtype == "bf16":
        return lambda: tkg.gemm_bf16(ops[0], ops[1], out=C, stream=stream)
    if dtype == "fp8":
        return lambda: tkg.gemm_fp8(ops[0], ops[1], ops[2], ops[3], out=C, stream=stream)
    return lambda: tkg.gemm_fp4_blockscaled(*ops, out=C, stream=stream)


def _roofline(kernel, tflops, peak, basis):
    """One roofline entry: achieved = algorithmic flops / event-timed launch
    duration; traffic and MFMA busy from the committed counter runs of the
    same kernel code (None once the kernels have changed since)."""
    return {"kernel": kernel, "bound": "mfma", "achieved": tflops, "peak": peak,
            "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "peak_basis": basis,
            "traffic": measured_traffic(kernel),
            "mfma_busy": measured(kernel, "mfma_busy_fraction"),
            "clock_ghz": measured(kernel, "clock_ghz_estimate")}


# Ablations of the dense kernels (page "ThunderKittens: Simple, Fast, and
# Adorable AI Kernels", section 3.4, Tables 1-3 and its section 5 note on
# the missing swizzle ablation; page "ThunderKittens reaches 22.4 PFLOPS on
# NVIDIA Rubin" for the release timing and ring depth). Each group:
# (group, dtype, M, N, K, [(setting label, tkg_gemm_ex options), ...]).
# Every setting computes the same bits at these sizes (the GPU tests check
# it; fp8's 16x16x128 and 32x32x64 blocks can round a few elements to
# neighbouring bf16 values once K reaches 16384).
def ablation_groups():
    # bf16 17 is the default's configuration on the interleaved schedule:
    # the ring-depth and MFMA-shape groups compare on that schedule
    ring = [("1 stage of 128 B (2 slots)", {"variant": 9}),
            ("2 stages of 128 B (4 slots)", {"variant": 17}),
            ("2.5 stages of 128 B (5 slots)", {"variant": 1}),
            ("2 stages of 128 B, early reads (default)", {"variant": 0}),
            ("2.5 stages of 128 B, early reads", {"variant": 18})]
    ring += [("%d stage%s of 64 B (32x32 blocks)" % (d, "s" if d > 1 else ""),
              {"variant": 9 + d}) for d in range(1, 6)]
    groups = [("ring_depth", "bf16", 4096, 4096, 4096, ring)]
    # operands of 1 GiB, four times the last-level cache: loads come from HBM
    groups.append(("ring_depth_large", "bf16", 16384, 16384, 16384, [
        ("2 stages of 128 B, early reads", {"variant": 0}),
        ("2.5 stages of 128 B, early reads (automatic)", {}),
        ("2.5 stages of 128 B, interleaved", {"variant": 1})]))
    for k in (64, 128, 256, 512, 1024):
        groups.append(("persistent", "bf16", 4096, 4096, k, [
            ("256x256 tiles, one workgroup per tile (256 = one per CU)", {"variant": 0}),
            ("128x128 tiles, persistent (2 per CU, 2 tiles each)", {"variant": 4}),
            ("128x128 tiles, one workgroup per tile (1024)", {"variant": 4, "grid": 1 << 20})]))
    groups.append(("order", "bf16", 16384, 16384, 16384, [
        ("XCD blocks, bands of 16 rows (automatic)", {}),
        ("grouped (GROUP_M 8) + XCD remap", {"group_m": 8, "xcd_remap": 1}),
        ("grouped (GROUP_M 8), no XCD remap", {"group_m": 8, "xcd_remap": 0}),
        ("row-major tile order + XCD remap", {"group_m": 1}),
        ("row-major tile order, no XCD remap (naive)", {"group_m": 1, "xcd_remap": 0})]))
    groups.append(("order", "fp8", 16384, 16384, 16384, [
        ("XCD blocks, bands of 32 rows (automatic)", {}),
        ("grouped (GROUP_M 8) + XCD remap", {"group_m": 8, "xcd_remap": 1}),
        ("grouped (GROUP_M 32), no XCD remap", {"group_m": 32, "xcd_remap": 0})]))
    for dt in ("bf16", "fp8"):
        groups.append(("swizzle", dt, 8192, 8192, 8192, [
            ("swizzled LDS (default)", {"variant": 0}),
            ("plain LDS rows (no swizzle)", {"variant": 6})]))
    groups.append(("schedule", "bf16", 8192, 8192, 8192, [
        ("early reads (default)", {"variant": 0}),
        ("interleaved", {"variant": 17}),
        ("early B-slab release", {"variant": 7}),
        ("ping-pong, 2 stages of 128 B", {"variant": 8}),
        ("ping-pong, 4 stages of 64 B", {"variant": 15})]))
    groups.append(("schedule", "fp8", 8192, 8192, 8192, [
        ("interleaved (default)", {"variant": 0}),
        ("early reads", {"variant": 11}),
        ("early B-slab release", {"variant": 7}),
        ("ping-pong, 2 stages of 128 B", {"variant": 8})]))
    groups.append(("mfma_shape", "bf16", 8192, 8192, 8192, [
        ("16x16x32, 8 waves", {"variant": 17}),
        ("32x32x16, 8 waves", {"variant": 2}),
        ("16x16x32, 4 waves (one per SIMD)", {"variant": 3}),
        ("16x16x32, 4 waves (one per SIMD), early reads", {"variant": 16})]))
    groups.append(("mfma_shape", "fp8", 8192, 8192, 8192, [
        ("32x32x64, 8 waves (default)", {"variant": 0}),
        ("16x16x128, 4 waves (one per SIMD)", {"variant": 2}),
        ("32x32x64, 4 waves (one per SIMD)", {"variant": 3}),
        ("32x32x64, 4 waves (one per SIMD), early reads", {"variant": 9})]))
    return groups


def run_ablations(args):
    """Every ablation setting as a block of warmup + timed launches (HIP
    events), rounds alternating over a group's settings; prints one JSON
    line with the results and the launch log, then the counter-calibration
    copies."""
    import numpy as np
    import torch

    import gemm_inputs.device as gdev
    import tiled_dense_gemm_amd as tkg

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    log = LaunchLog(stream)
    rows = []
    for gi_, (group, dtype, M, N, K, settings) in enumerate(ablation_groups()):
        ops = _operands(gdev, dtype, M, N, K, 1.0 if dtype == "fp8" else None, dev, 40)
        if dtype == "bf16":
            A, B, sa, sb, d = ops[0], ops[1], 1.0, 1.0, tkg.DTYPE_BF16
        else:
            A, sa, B, sb, d = ops[0], ops[1], ops[2], ops[3], tkg.DTYPE_FP8
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        res = {lab: [] for lab, _ in settings}
        for rnd in range(args.ablation_rounds):
            for lab, opt in settings:
                def fn(opt=opt):
                    st = tkg.tkg_gemm_ex(d, M, N, K, A, None, sa, B, None, sb, C, stream=stream,
                                         **opt)
                    assert st == 0, (group, lab, st)
                r = log.time("%d|%s|%s|%d" % (gi_, group, lab, rnd), "gemm_" + dtype, fn,
                             args.warmup, args.steps)
                res[lab].append(r["ms_mean"])
        for lab, opt in settings:
            ms = float(np.median(res[lab]))
            rows.append({"gid": gi_, "group": group, "dtype": dtype, "M": M, "N": N, "K": K,
                         "setting": lab, "options": opt, "ms_mean_per_round": res[lab],
                         "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)})
        del ops, A, B, C
        torch.cuda.empty_cache()
    # calibration copies (1 GiB read + 1 GiB written each) for the byte counters
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"ablations": rows, "kernel_source_hash": kernel_source_hash(),
                      "steps": args.steps, "warmup": args.warmup,
                      "rounds": args.ablation_rounds, "launch_log": log.blocks}), flush=True)
    return 0


def summarize_ablations(run_dirs, out_md, out_json, command):
    """profiles/ablations.md from rocprofv3 passes over `bench.py
    --ablations`: each run dir holds one pass (a --kernel-trace run or a
    --pmc run) and the log of the bench run it traced (run.log); every
    dispatch is attributed to its setting through that run's launch log."""
    import csv
    import glob
    import statistics

    def rows(d, pattern):
        out = []
        for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    def line_of(d):
        for l in open(os.path.join(d, "run.log")):
            if l.startswith("{") and '"ablations"' in l:
                return json.loads(l)
        raise SystemExit("no ablation line in %s/run.log" % d)

    def split(seq, blocks):
        """{block name: [rows of its timed launches]} by dispatch order."""
        out, pos = {}, {}
        for b in blocks:
            i = pos.get(b["key"], 0)
            out[b["name"]] = seq.get(b["key"], [])[i + b["warmup"]:i + b["warmup"] + b["timed"]]
            pos[b["key"]] = i + b["warmup"] + b["timed"]
        return out

    trace = {}
    counters = {}
    calib = {}
    ref = None
    for d in run_dirs:
        bl = line_of(d)
        ref = ref or bl
        tr = rows(d, "*kernel_trace.csv")
        if tr:
            seq = {}
            for r in sorted(tr, key=lambda r: int(r["Start_Timestamp"])):
                k = _kernel_key(r["Kernel_Name"])
                if k:
                    seq.setdefault(k, []).append(
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
            for name, ds in split(seq, bl["launch_log"]).items():
                trace.setdefault(name.rsplit("|", 1)[0], []).extend(ds)
        cc = rows(d, "*counter_collection.csv")
        if cc:
            by_disp = {}
            for r in cc:
                by_disp.setdefault(int(r["Dispatch_Id"]), []).append(r)
            seq = {}
            for disp in sorted(by_disp):
                rs = by_disp[disp]
                k = _kernel_key(rs[0]["Kernel_Name"])
                vals = {r["Counter_Name"]: float(r["Counter_Value"]) for r in rs}
                if k:
                    seq.setdefault(k, []).append(vals)
                elif "copy" in rs[0]["Kernel_Name"]:
                    for c, v in vals.items():
                        if v > 512 * 1024:
                            calib.setdefault(c, []).append(v)
            for name, vs in split(seq, bl["launch_log"]).items():
                key = name.rsplit("|", 1)[0]
                for vals in vs:
                    for c, v in vals.items():
                        counters.setdefault(key, {}).setdefault(c, []).append(v)
    gib_kib = 1024.0 * 1024.0
    fac = {c: gib_kib / statistics.mean(v) for c, v in calib.items()}
    rec = {"kernel_source_hash": ref["kernel_source_hash"], "command": command,
           "calibration": fac, "rows": []}
    lines = ["# Ablations of the dense GEMM kernels on one MI355X (rocprofv3)", "",
             "Every setting computes the same bits at these sizes (the GPU tests compare "
             "all kernel configurations and launch options bit for bit; fp8's 16x16x128 "
             "and 32x32x64 blocks can round a few elements to neighbouring bf16 values "
             "once K reaches 16384). Kernel source hash %s."
             % ref["kernel_source_hash"], "", "Produced by:", "", "```", command, "```", "",
             "Columns: TFLOP/s from the HIP-event mean of the traced run (median over %d "
             "alternating rounds of %d launches after %d warmup launches) and from the "
             "kernel trace's durations of the same launches; MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over SQ_BUSY_CYCLES / %d shader engines; "
             "clock = SQ_BUSY_CYCLES / %d over the traced duration; LDS conflict = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; HBM bytes = FETCH_SIZE x %s + "
             "WRITE_SIZE x %s (KiB, calibrated by 1 GiB copies); L2 hit = TCC_HIT / (HIT + "
             "MISS)." % (ref["rounds"], ref["steps"], ref["warmup"], SHADER_ENGINES, SHADER_ENGINES,
                         "%.3f" % fac.get("FETCH_SIZE", float("nan")),
                         "%.3f" % fac.get("WRITE_SIZE", float("nan"))), ""]
    cur = None
    for row in ref["ablations"]:
        gkey = "%d|%s|%s" % (row["gid"], row["group"], row["setting"])
        head = (row["group"], row["dtype"], row["M"], row["N"], row["K"])
        if head != cur:
            cur = head
            lines += ["", "## %s, %s, M=%d N=%d K=%d" % head, "",
                      "| setting | TFLOP/s (events) | TFLOP/s (trace) | trace mean us | "
                      "MFMA busy | clock GHz | LDS conflict | HBM bytes | L2 hit |",
                      "|---|---|---|---|---|---|---|---|---|"]
        ds = trace.get(gkey, [])
        cs = counters.get(gkey, {})
        flops = 2.0 * row["M"] * row["N"] * row["K"]
        mean_us = statistics.mean(ds) if ds else None
        g = lambda c: statistics.mean(cs[c]) if cs.get(c) else None
        act = _active_cycles(cs)
        busy = (g("SQ_VALU_MFMA_BUSY_CYCLES") / 1024.0 / act
                if g("SQ_VALU_MFMA_BUSY_CYCLES") and act else None)
        ghz = act / (mean_us * 1e3) if act and mean_us else None
        confl = (g("SQ_LDS_BANK_CONFLICT") / max(1.0, g("SQ_LDS_IDX_ACTIVE"))
                 if g("SQ_LDS_BANK_CONFLICT") is not None and g("SQ_LDS_IDX_ACTIVE") else None)
        hbm = (g("FETCH_SIZE") * 1024 * fac["FETCH_SIZE"] + g("WRITE_SIZE") * 1024 * fac["WRITE_SIZE"]
               if g("FETCH_SIZE") and g("WRITE_SIZE") and "FETCH_SIZE" in fac and
               "WRITE_SIZE" in fac else None)
        l2 = (g("TCC_HIT_sum") / (g("TCC_HIT_sum") + g("TCC_MISS_sum"))
              if g("TCC_HIT_sum") and g("TCC_MISS_sum") is not None else None)
        out = dict(row, trace_mean_us=mean_us,
                   trace_tflops=flops / (mean_us * 1e-6) / 1e12 if mean_us else None,
                   mfma_busy=busy, clock_ghz=ghz, lds_conflict_over_active=confl,
                   hbm_bytes=hbm, l2_hit_rate=l2)
        rec["rows"].append(out)
        f = lambda v, fmt: fmt % v if v is not None else "-"
        lines.append("| %s | %.1f | %s | %s | %s | %s | %s | %s | %s |" % (
            row["setting"], row["tflops"], f(out["trace_tflops"], "%.1f"), f(mean_us, "%.1f"),
            f(busy, "%.3f"), f(ghz, "%.2f"), f(confl, "%.4f"),
            f(hbm, "%.3g"), f(l2, "%.3f")))
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
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU budget of the oracle baseline when the whole bf16 "
                         "product would take longer than 45 s")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the timed sweep over the other configurations")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--summarize-profile", nargs=3,
                    metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--profile-command", default="")
    ap.add_argument("--bench-log", default=None,
                    help="log of the traced bench run (its JSON line gives the launch "
                         "log and the HIP-event means)")
    ap.add_argument("--summarize-attn-profile", nargs=3,
                    metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--with-attn", action="store_true",
                    help="time attention forward on its workloads under next_rows "
                         "(the default; kept for older command lines)")
    ap.add_argument("--with-mx", action="store_true",
                    help="time the MX products under next_rows (the default; kept "
                         "for older command lines)")
    ap.add_argument("--ablations", action="store_true",
                    help="run the dense-kernel ablations instead of the step (one JSON "
                         "line; for rocprofv3 passes)")
    ap.add_argument("--ablation-rounds", type=int, default=2)
    ap.add_argument("--summarize-ablations", nargs="+", metavar="RUN_DIR",
                    help="rocprofv3 pass directories of --ablations runs (each with its "
                         "run.log) -> profiles/ablations.md")
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

    if args.summarize_ablations:
        return summarize_ablations(args.summarize_ablations,
                                   os.path.join(ROOT, "profiles", "ablations.md"),
                                   os.path.join(ROOT, "profiles", "ablations.json"),
                                   args.profile_command)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (a GEMM shards by splitting N across GPUs with no "
              "exchange; the per-GPU kernel is the one measured here).",
              file=sys.stderr)
        return 2

    import torch

    import gemm_inputs.device as gdev
    import tiled_dense_gemm_amd as tkg

    assert torch.cuda.is_available(), "bench.py needs the HIP device"
    if args.ablations:
        return run_ablations(args)
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
    log = LaunchLog(stream)

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

    # ---- the step: the three products back to back, K times -------------
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
    for k in names:
        log.blocks.append({"name": "step_" + k, "key": "gemm_" + k,
                           "warmup": args.warmup, "timed": args.steps})

    import numpy as np
    per = {k: [] for k in names}
    for s in range(args.steps):
        for i, k in enumerate(names):
            per[k].append(ev[s][i].elapsed_time(ev[s][i + 1]))
    step_ms = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(args.steps)) / args.steps
    kernels = {}
    for k in names:
        ms = float(np.mean(per[k]))
        peak = PEAK_TFLOPS[k]
        kernels["gemm_" + k] = dict(
            {"ms_mean": round(ms, 4), "ms_min": round(float(np.min(per[k])), 4),
             "ms_median": round(float(np.median(per[k])), 4)},
            **_rate(flops, ms, peak))
    k4 = kernels["gemm_fp4_blockscaled"]
    k4["peak_basis"] = "fp16 MFMA rate, the instruction the exact dequantized path issues"
    k4["frac_of_fp4_dense_peak"] = round(k4["tflops"] / PEAK_FP4_DENSE, 4)
    value = len(names) * flops / (step_ms * 1e-3) / 1e12

    headline = {
        "bf16": {"tflops": kernels["gemm_bf16"]["tflops"],
                 "frac_of_dense_peak": kernels["gemm_bf16"]["frac_of_peak"],
                 "dense_peak_tflops": PEAK_TFLOPS["bf16"]},
        "fp8": {"tflops": kernels["gemm_fp8"]["tflops"],
                "frac_of_dense_peak": kernels["gemm_fp8"]["frac_of_peak"],
                "dense_peak_tflops": PEAK_TFLOPS["fp8"]},
        "workload": "M=N=K=%d, ms mean over %d timed launches after %d warmup steps"
                    % (n, args.steps, args.warmup)}

    rooflines = [
        _roofline("gemm_bf16", kernels["gemm_bf16"]["tflops"], PEAK_TFLOPS["bf16"],
                  "bf16 dense MFMA"),
        _roofline("gemm_fp8", kernels["gemm_fp8"]["tflops"], PEAK_TFLOPS["fp8"],
                  "fp8 dense MFMA"),
        _roofline("gemm_fp4_blockscaled", k4["tflops"], PEAK_TFLOPS["fp4_blockscaled"],
                  "fp16 dense MFMA (the instruction the exact path issues)"),
        _roofline("gemm_fp4_blockscaled", k4["tflops"], PEAK_FP4_DENSE, "fp4 dense MFMA"),
    ]
    # the contract's roofline: the step's dominant (longest) kernel
    dom = max(names, key=lambda k: kernels["gemm_" + k]["ms_mean"])
    roofline = dict(rooflines[names.index(dom)])

    # ---- the other configurations, each on its own operands -------------
    configs = None
    if not args.no_configs:
        configs = {}
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        DTYPE_CODES = {"bf16": tkg.DTYPE_BF16, "fp8": tkg.DTYPE_FP8,
                       "fp4_blockscaled": tkg.DTYPE_FP4_BLOCKSCALED}
        for cname, dtype, cm, cn, ck, std, cw, cs in CONFIGS:
            ops = _operands(gdev, dtype, cm, cn, ck, std, dev, 30)
            Cc = torch.empty((cm, cn), dtype=torch.bfloat16, device=dev)
            torch.cuda.synchronize()
            r = log.time(cname, "gemm_" + dtype, _call(tkg, dtype, ops, Cc, stream), cw, cs)
            cf = 2.0 * cm * cn * ck
            row = {"dtype": dtype, "M": cm, "N": cn, "K": ck}
            row.update(r)
            row.update(_rate(cf, r["ms_mean"], PEAK_TFLOPS[dtype]))
            if dtype == "fp4_blockscaled":
                row["frac_of_fp4_dense_peak"] = round(row["tflops"] / PEAK_FP4_DENSE, 4)
            # the launch the automatic options made (configuration, grid,
            # tile order), as the library plans it for this device
            row["plan"] = tkg.plan_launch(DTYPE_CODES[dtype], cm, cn, ck, cus=cus)
            configs[cname] = row
            del ops, Cc
            torch.cuda.empty_cache()

    # ---- next rows: the MX products and attention, outside the step -----
    next_rows = None
    if extra:
        next_rows = {}
        for k, fn in extra.items():
            r = log.time("next_" + k, "gemm_" + k, fn, args.warmup, args.steps)
            next_rows["gemm_" + k] = dict(r, **_rate(flops, r["ms_mean"], PEAK_MX_TFLOPS[k]))
    if args.with_attn:
        next_rows = next_rows or {}
        next_rows.update(time_attention(args, dev, stream))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(((A16, B16), (A8, sa, B8, sb), (A4, As4, ta, B4, Bs4, tb)),
                           args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s",
        "headline": headline,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+fp8+fp4",
        "data": "synthetic",
        "config": {"workload": "one step = C = A*B at M=N=K=%d in bf16 (A, B ~ N(0,1)/sqrt(K)), "
                               "fp8 e4m3 with per-tensor amax/448 scales, and block-scaled "
                               "e2m1 (e4m3 scale per 16, fp32 tensor scale), back to back; "
                               "value = the step's 3 x 2MNK flops over its time; "
                               "A row-major, B column-major, bf16 C" % n,
                   "M": M, "N": N, "K": K, "global_batch": 1, "seq_len": None,
                   "parallelism": "single GPU"},
        "device": _device_description(tkg, dev),
        "kernels": kernels,
        "roofline": roofline,
        "rooflines": rooflines,
        "cpu_baseline": cpu,
        "configs": configs,
        "wall_s_timed": round(wall, 3),
        "launch_log": log.blocks,
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


def _device_description(tkg, dev):
    """The GPU the run used: name, architecture, compute units and the
    runtime's peak shader clock (the clock the published dense peaks
    assume; the kernels' measured clocks are in `rooflines`)."""
    import torch
    props = torch.cuda.get_device_properties(dev)
    info = tkg.device_info()
    return {"name": props.name, "arch": props.gcnArchName, "cus": info["cus"],
            "peak_clock_mhz": info["peak_clock_mhz"]}


def _host_description():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": affinity,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(ops, seconds, full_limit_s=45.0):
    """The oracle (its decode of each format and its plain fp64 C product,
    OpenMP over rows) on the step's products. bf16: the whole 8192^3
    product, in row panels (R rows of A against all columns of B, full K:
    the loop the full product runs), when a first panel predicts it within
    `full_limit_s`; otherwise panels until `seconds` and the full time
    extrapolated (the loop is latency-bound on the in-order fp64 sum, so the
    rate does not depend on R). fp8 and 4-bit: row panels for about a tenth
    of `seconds` each, the full time extrapolated. value: the bf16 rate."""
    import numpy as np
    import torch

    import oracle

    def rows(x, r0, r1):
        t = x[r0:r1]
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    (A16, B16), (A8, sa, B8, sb), (A4, As4, ta, B4, Bs4, tb) = ops
    M, K = A16.shape
    N = B16.shape[0]
    full = {"bf16": (rows(B16, 0, N),), "fp8": (rows(B8, 0, N),),
            "fp4_blockscaled": (rows(B4, 0, N), rows(Bs4, 0, N))}

    def panel(name, r0, r1):
        if name == "bf16":
            args, fn = (rows(A16, r0, r1), full[name][0]), oracle.gemm_bf16
        elif name == "fp8":
            args, fn = (rows(A8, r0, r1), sa, full[name][0], sb), oracle.gemm_fp8
        else:
            args = (rows(A4, r0, r1), rows(As4, r0, r1), ta, full[name][0], full[name][1], tb)
            fn = oracle.gemm_fp4_blockscaled
        t = time.perf_counter()
        fn(*args)
        return time.perf_counter() - t

    per = {}
    for name in ("bf16", "fp8", "fp4_blockscaled"):
        budget = seconds if name == "bf16" else seconds / 10.0
        done_rows, used, r = 0, 0.0, 64
        whole = False
        while done_rows < M:
            r = min(r, M - done_rows)
            used += panel(name, done_rows, done_rows + r)
            done_rows += r
            predicted = used / done_rows * M
            if name == "bf16" and predicted <= full_limit_s:
                whole = True
                r = 1024
                continue
            if used >= budget:
                break
            r *= 2
        rate = 2.0 * done_rows * N * K / used / 1e12
        per[name] = {"tflops": round(rate, 5), "rows": done_rows, "seconds": round(used, 2),
                     "whole_product": whole and done_rows == M,
                     "full_product_s": round(used if done_rows == M else
                                             2.0 * M * N * K / (rate * 1e12), 1)}
    b = per["bf16"]
    return {"value": b["tflops"], "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": ("the whole %dx%dx%d bf16 product (%.1f s)" % (M, N, K, b["seconds"])
                       if b["whole_product"] else
                       "%d of %d rows of the %dx%dx%d bf16 product, full width and K "
                       "(%.1f s; full time extrapolated)" % (b["rows"], M, M, N, K, b["seconds"]))
                      + "; fp8 and block-scaled 4-bit: full-width row panels (%d and %d rows), "
                        "full time extrapolated; the oracle's decode and plain fp64 C product "
                        "on its OpenMP threads" % (per["fp8"]["rows"],
                                                   per["fp4_blockscaled"]["rows"]),
            "per_dtype": per, "host": _host_description()}


if __name__ == "__main__":
    sys.exit(main())
