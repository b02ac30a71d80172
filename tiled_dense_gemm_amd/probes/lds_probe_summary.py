"""Join the LDS bank probe's pattern list with its rocprofv3 counters.

Usage:
    python lds_probe_summary.py PROBE_STDOUT COUNTER_DIR GOLDEN_JSON SUMMARY_MD COMMAND

PROBE_STDOUT: what lds_bank_probe printed ("pattern <id> <bytes> <op>
<name> : <addresses>", op r = ds_read, w = ds_write, one line per dispatch,
in dispatch order); COUNTER_DIR: the
rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE output directory.
Per dispatch, conflict degree = 1 / (1 - SQ_LDS_BANK_CONFLICT /
SQ_LDS_IDX_ACTIVE), rounded. Writes the measured table as JSON (read by
tests/test_bank_model.py) and a Markdown summary.
"""
from __future__ import annotations

import collections
import csv
import glob
import json
import os
import sys


def main(argv) -> int:
    probe_out, counter_dir, golden, summary, command = argv[1:6]
    pats = []
    for line in open(probe_out):
        if not line.startswith("pattern "):
            continue
        head, addrs = line.rstrip("\n").split(" : ") if " : " in line else line.rstrip("\n").split(" :")
        _, pid, nbytes, op, name = head.split(" ", 4)
        pats.append({"id": int(pid), "bytes": int(nbytes), "op": op, "name": name,
                     "addresses": [int(a) for a in addrs.split()]})
    per = collections.defaultdict(dict)
    for f in glob.glob(os.path.join(counter_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "lds_probe" not in r["Kernel_Name"]:
                continue
            per[int(r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
    dispatches = sorted(per)
    if len(dispatches) != len(pats):
        print("dispatch count %d != pattern count %d" % (len(dispatches), len(pats)))
        return 1
    for p, d in zip(pats, dispatches):
        c = per[d]
        ratio = c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"])
        p["conflict_over_active"] = round(ratio, 4)
        p["degree"] = int(round(1.0 / (1.0 - ratio))) if ratio < 0.999 else 999
    rec = {"source": "measured on one MI355X (gfx950) with "
                     "tiled_dense_gemm_amd/probes/lds_bank_probe.hip; per dispatch "
                     "degree = 1 / (1 - SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)",
           "command": command,
           "patterns": [p for p in pats if not p["name"].startswith("search ")],
           "search_16x16_degrees": [p["degree"] for p in pats if p["name"].startswith("search ")]}
    json.dump(rec, open(golden, "w"), indent=None, separators=(",", ":"))
    lines = ["# LDS bank conflicts on gfx950 (MI355X), measured", "", "Produced by:", "",
             "```", command, "```", "",
             "Per dispatch, conflict degree = 1 / (1 - SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE). "
             "Address lists: `tests/golden/lds_probe_gfx950.json`.", "",
             "| pattern | op | bytes/lane | conflict / active | degree |", "|---|---|---|---|---|"]
    for p in rec["patterns"]:
        if " frag " in p["name"] and not p["name"].endswith(" frag 0"):
            continue
        lines.append("| %s | %s | %d | %.3f | %d |" % (p["name"], "write" if p["op"] == "w" else "read",
                                                      p["bytes"], p["conflict_over_active"], p["degree"]))
    kern = [p for p in rec["patterns"] if " frag " in p["name"]]
    for kind in ("bf16 16x16x32", "fp8 32x32x64", "fp8 16x16x128", "4-bit values"):
        for sw in ("swizzled", "unswizzled"):
            ds = [p["degree"] for p in kern if p["name"].startswith(kind + " " + sw)]
            lines.append("")
            lines.append("%s %s fragment reads: %d patterns, degrees %s" % (
                kind, sw, len(ds), sorted(collections.Counter(ds).items())))
    s = rec["search_16x16_degrees"]
    lines += ["", "Linear row swizzles of 128-byte rows (chunk ^ A*bits(row mod 16), 4096 "
              "candidates) read with the 16x16 fragment pattern: degree histogram %s." % (
                  sorted(collections.Counter(s).items()),), ""]
    open(summary, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
