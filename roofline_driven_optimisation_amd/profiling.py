"""Summaries of rocprofv3 CSV output (kernel statistics and HBM counters).

Used to turn a profiling run of ``bench.py`` into the short text summaries
kept beside the benchmark.  Two inputs:

* ``--kernel-trace --stats --output-format csv`` writes ``*_kernel_stats.csv``
  (per-kernel call count and durations);
* ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` with ``--output-format csv``
  write ``*_counter_collection.csv`` (one row per dispatch, values in KiB).

HBM bytes per launch = median counter value x the calibration factor, where
the factor makes a plain device copy of known size read and write exactly
its size (counters are taken below L2, so MALL hits count as fabric traffic).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import re
import os
import statistics
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))

KERNEL_SOURCES = {
    "bf16_mfma": "bf16_mfma.hip",
    "bf16_pp": "bf16_mfma.hip",
    "bf16_q4": "bf16_mfma.hip",
    "f32_mfma": "f32_mfma.hip",
    "f32_dma": "f32_mfma.hip",
    "skinny": "skinny_bf16.hip",
    "naive": "naive.hip",
}


def code_hash(text: str) -> str:
    """sha256[:16] of C++/HIP source with comments, trailing blanks and empty
    lines removed, so that editing a comment does not mark a measurement of
    the code as stale.  (The sources hold no string literal containing
    comment markers.)"""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines()]
    code = "\n".join(line for line in lines if line)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def source_hash(kernel_family: str) -> str:
    """code_hash of the source that defines a kernel family."""
    for prefix, fname in KERNEL_SOURCES.items():
        if kernel_family.startswith(prefix):
            with open(os.path.join(HERE, "csrc", fname)) as f:
                return code_hash(f.read())
    return ""


def short_name(name: str) -> str:
    """'void mgemm::(anonymous namespace)::bf16_mfma_kernel<256, 256, false>(...)'
    -> 'bf16_mfma_kernel<256, 256, false>'."""
    base = name.split("(")[0] if "(anonymous namespace)" not in name else \
        name.split("::")[-1].split("(")[0]
    if "(anonymous namespace)" in name:
        tail = name.split("(anonymous namespace)::", 1)[1]
        depth, out = 0, []
        for ch in tail:
            if ch == "(" and depth == 0:
                break
            depth += ch == "<"
            depth -= ch == ">"
            out.append(ch)
        base = "".join(out)
    return base.replace("void ", "").strip()


def kernel_stats(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3,
                         "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                         "pct": float(r["Percentage"])})
    return rows


def dispatch_stats(path: str):
    """Per (kernel, grid size) statistics from a ``*_kernel_trace.csv``: one
    kernel launched on several shapes shows up once per launch shape."""
    acc = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            acc[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in acc.values())
    rows = []
    for (k, grid, wg), v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        rows.append({"kernel": "%s [%d workgroups x %d]" % (k, grid // max(wg, 1), wg),
                     "calls": len(v), "avg_us": statistics.mean(v), "min_us": min(v),
                     "max_us": max(v), "pct": 100.0 * sum(v) / total})
    return rows


def counter_medians(path: str):
    """{(kernel, counter): median value (KiB per dispatch)}; a kernel launched
    on several shapes is keyed as 'name [W workgroups]' per launch shape."""
    acc = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            wg = max(int(r.get("Workgroup_Size", 1) or 1), 1)
            grid = int(r.get("Grid_Size", 0) or 0)
            name = "%s [%d workgroups]" % (short_name(r["Kernel_Name"]), grid // wg)
            acc[(name, r["Counter_Name"])].append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in acc.items()}


NUM_XCD = 8          # GRBM counters are summed over the XCDs
NUM_SIMD = 256 * 4   # MFMA busy cycles are summed over every SIMD
SPEC_CLOCK_GHZ = 2.4
MOPS_FLOP = 512      # one MFMA "MOP" is 512 floating-point operations


def mfma_rows(path: str):
    """Per kernel and launch shape, from one --pmc pass with GRBM_GUI_ACTIVE,
    SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_* (medians over
    dispatches): duration, average shader clock, share of SIMD cycles the
    matrix cores were busy, and the MFMA FLOPs counted."""
    acc = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            wg = max(int(r.get("Workgroup_Size", 1) or 1), 1)
            grid = int(r.get("Grid_Size", 0) or 0)
            name = "%s [%d workgroups]" % (short_name(r["Kernel_Name"]), grid // wg)
            acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                acc[name]["_ns"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    rows = []
    for name, c in sorted(acc.items()):
        if "GRBM_GUI_ACTIVE" not in c or not any(c["SQ_VALU_MFMA_BUSY_CYCLES"]):
            continue
        med = {k: statistics.median(v) for k, v in c.items()}
        cycles = med["GRBM_GUI_ACTIVE"] / NUM_XCD
        ns = med["_ns"]
        mops = sum(v for k, v in med.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS"))
        rows.append({"kernel": name, "us": ns / 1e3, "clock_ghz": cycles / ns,
                     "mfma_busy": med["SQ_VALU_MFMA_BUSY_CYCLES"] / (NUM_SIMD * cycles),
                     "mfma_gflop": mops * MOPS_FLOP / 1e9,
                     "mfma_tflops": mops * MOPS_FLOP / ns / 1e3})
    return rows


def mfma_markdown(rows) -> str:
    out = ["| kernel | us | avg clock GHz | MFMA busy (of SIMD cycles) | MFMA GFLOP counted | "
           "TFLOP/s from counters | share of spec (busy x clock / 2.4 GHz) |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %.1f | %.2f | %.1f %% | %.1f | %.1f | %.1f %% |" % (
            r["kernel"], r["us"], r["clock_ghz"], 100 * r["mfma_busy"], r["mfma_gflop"],
            r["mfma_tflops"], 100 * r["mfma_busy"] * r["clock_ghz"] / SPEC_CLOCK_GHZ))
    return "\n".join(out)


def stats_markdown(rows) -> str:
    out = ["| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %d | %.1f | %.1f | %.1f | %.2f |" % (
            r["kernel"], r["calls"], r["avg_us"], r["min_us"], r["max_us"], r["pct"]))
    return "\n".join(out)


def _find(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, d))
    return hits[0]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats", help="markdown table from a --kernel-trace --stats run")
    s.add_argument("dir")
    t = sub.add_parser("trace", help="markdown table per kernel and launch shape from "
                       "--kernel-trace output")
    t.add_argument("dir")
    m = sub.add_parser("mfma", help="clock and matrix-core utilisation from a --pmc pass "
                       "with GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_*")
    m.add_argument("dir")
    c = sub.add_parser("counters", help="calibrated HBM bytes per dispatch")
    c.add_argument("--fetch", required=True, help="dir of the FETCH_SIZE run")
    c.add_argument("--write", required=True, help="dir of the WRITE_SIZE run")
    c.add_argument("--copy-fetch", required=True, help="dir of the copy probe's FETCH_SIZE run")
    c.add_argument("--copy-write", required=True, help="dir of the copy probe's WRITE_SIZE run")
    c.add_argument("--copy-mib", type=float, required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        print(stats_markdown(kernel_stats(_find(args.dir, "_kernel_stats.csv"))))
        return
    if args.cmd == "mfma":
        print(mfma_markdown(mfma_rows(_find(args.dir, "_counter_collection.csv"))))
        return
    if args.cmd == "trace":
        print(stats_markdown(dispatch_stats(_find(args.dir, "_kernel_trace.csv"))))
        return
    fetch = counter_medians(_find(args.fetch, "_counter_collection.csv"))
    write = counter_medians(_find(args.write, "_counter_collection.csv"))
    cf = counter_medians(_find(args.copy_fetch, "_counter_collection.csv"))
    cw = counter_medians(_find(args.copy_write, "_counter_collection.csv"))
    kib = args.copy_mib * 1024
    f_fac = kib / max(v for (k, n), v in cf.items() if n == "FETCH_SIZE")
    w_fac = kib / max(v for (k, n), v in cw.items() if n == "WRITE_SIZE")
    print("calibration: copy of %.0f MiB -> FETCH_SIZE factor %.3f, WRITE_SIZE factor %.3f"
          % (args.copy_mib, f_fac, w_fac))
    for (k, n), v in sorted(fetch.items()):
        w = write.get((k, "WRITE_SIZE"), float("nan"))
        fb, wb = v * 1024 * f_fac, w * 1024 * w_fac
        print("%s: fetch %.1f MB, write %.1f MB, total %.1f MB per dispatch (source %s)"
              % (k, fb / 1e6, wb / 1e6, (fb + wb) / 1e6, source_hash(k.split("<")[0])))


if __name__ == "__main__":
    main()
