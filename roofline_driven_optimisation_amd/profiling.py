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
    "bf16_q16": "bf16_mfma.hip",
    "f32_mfma": "f32_mfma.hip",
    "f32_dma": "f32_mfma.hip",
    "skinny": "skinny_bf16.hip",
    "naive": "naive.hip",
    "fp8_q4": "bf16_mfma.hip",
    "fp8_wide": "bf16_mfma.hip",
    "reduce": "reduce.hip",
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


# bench.py's phase markers: K = 0 GEMMs, one workgroup just before a timed
# loop and two just after it
MARKER_KERNEL = "scale_kernel"


def _marker_index(runs, i, workgroups):
    return (0 <= i < len(runs) and runs[i][0][0].startswith(MARKER_KERNEL) and
            runs[i][0][1] == workgroups)


def dispatch_stats(path: str, last: int = 0, gap_ms: float = 0.0, timed: bool = False):
    """Statistics from a ``*_kernel_trace.csv``, one row per run of
    consecutive dispatches of one kernel with one launch shape (a benchmark
    times its workloads one after another, so two workloads that launch the
    same kernel on the same grid still come out as separate rows, in time
    order).  With ``last`` > 0 only runs of at least ``last`` dispatches are
    reported, each by its last ``last`` dispatches: the timed, steady-state
    launches of each workload, not the warm-up or the copies between them.
    With ``gap_ms`` > 0 a run also ends where the device sat idle longer
    than that between two dispatches (a pause on the host, such as the end
    of a timed loop).  With ``timed`` only the runs that bench.py's phase
    markers enclose (a one-workgroup K = 0 launch before, a two-workgroup
    one after) are reported, whole: exactly the timed launches of each
    workload."""
    with open(path) as f:
        rows_in = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    prev_end = None
    for r in rows_in:
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        start, end = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        us = (end - start) / 1e3
        idle = gap_ms > 0 and prev_end is not None and start - prev_end > gap_ms * 1e6
        prev_end = end if prev_end is None else max(prev_end, end)
        if runs and runs[-1][0] == key and not idle:
            runs[-1][1].append(us)
        else:
            runs.append((key, [us]))
    if timed:
        shaped = [((k[0], k[1] // max(k[2], 1)), v) for k, v in runs]
        runs = [runs[i] for i in range(len(runs))
                if not shaped[i][0][0].startswith(MARKER_KERNEL) and
                _marker_index(shaped, i - 1, 1) and _marker_index(shaped, i + 1, 2)]
    if last > 0:
        runs = [(k, v[-last:]) for k, v in runs if len(v) >= last]
    total = sum(sum(v) for _, v in runs)
    rows = []
    for (k, grid, wg), v in runs:
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


NUM_SIMD = 256 * 4   # MFMA busy cycles are summed over every SIMD
SPEC_CLOCK_GHZ = 2.4
MOPS_FLOP = 512      # one MFMA "MOP" is 512 floating-point operations


def mfma_rows(path: str, last: int = 0):
    """Per kernel and launch shape, from one --pmc pass with
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_* (BF16, F8, F32),
    SQ_WAVE_CYCLES, SQ_WAIT_INST_ANY and SQ_WAIT_INST_LDS (medians over the
    last ``last`` dispatches, all if 0): the dispatch time, the MFMA FLOPs
    counted, the matrix cores' busy cycles per SIMD, and the share of wave
    cycles spent waiting (on any dependency; on LDS).  The shader clock is
    not derived from counters here: the steady-state clock comes from
    amd-smi samples (bench.py --sustain)."""
    acc = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        rows_in = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    for r in rows_in:
        wg = max(int(r.get("Workgroup_Size", 1) or 1), 1)
        grid = int(r.get("Grid_Size", 0) or 0)
        name = "%s [%d workgroups]" % (short_name(r["Kernel_Name"]), grid // wg)
        acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        if r["Counter_Name"] == "SQ_WAVE_CYCLES":
            acc[name]["_ns"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    rows = []
    for name, c in sorted(acc.items()):
        if not any(c.get("SQ_VALU_MFMA_BUSY_CYCLES", [])):
            continue
        if last > 0:
            c = {k: v[-last:] for k, v in c.items()}
        med = {k: statistics.median(v) for k, v in c.items() if v}
        mops = sum(v for k, v in med.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS"))
        wave = med.get("SQ_WAVE_CYCLES", float("nan"))
        rows.append({"kernel": name, "us": med["_ns"] / 1e3,
                     "mfma_gflop": mops * MOPS_FLOP / 1e9,
                     "busy_per_simd": med["SQ_VALU_MFMA_BUSY_CYCLES"] / NUM_SIMD,
                     "wait_any": med.get("SQ_WAIT_INST_ANY", float("nan")) / wave,
                     "wait_lds": med.get("SQ_WAIT_INST_LDS", float("nan")) / wave})
    return rows


def counter_runs(paths, labels, last: int = 8,
                 kernels=("bf16_q4", "bf16_q16", "bf16_mfma", "fp8_q4", "fp8_wide")):
    """Median counter values per workload from one or more --pmc passes of
    the same bench command: each pass's dispatches are split into runs of
    consecutive dispatches of one kernel and launch shape (one run per
    workload, as in dispatch_stats; where bench.py's phase markers are
    present, only the timed runs they enclose), runs of the named kernel families with
    at least 5 dispatches are matched in order to ``labels``, and every
    counter is the median over the last ``last`` dispatches of its run
    (summed over the device).  Returns {label: {counter: value, "us": ...}}."""
    out = {}
    for path in paths:
        with open(path) as f:
            rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
        disp, order = {}, []
        for r in rows:
            d = r.get("Dispatch_Id") or r["Start_Timestamp"]
            if d not in disp:
                wg = max(int(r.get("Workgroup_Size", 1) or 1), 1)
                disp[d] = {"key": (short_name(r["Kernel_Name"]),
                                   int(r.get("Grid_Size", 0) or 0) // wg),
                           "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3}
                order.append(d)
            disp[d][r["Counter_Name"]] = disp[d].get(r["Counter_Name"], 0.0) + float(
                r["Counter_Value"])
        runs = []
        for d in order:
            k = disp[d]["key"]
            if runs and runs[-1][0] == k:
                runs[-1][1].append(disp[d])
            else:
                runs.append((k, [disp[d]]))
        enclosed = [runs[i] for i in range(len(runs))
                    if not runs[i][0][0].startswith(MARKER_KERNEL) and
                    _marker_index(runs, i - 1, 1) and _marker_index(runs, i + 1, 2)]
        if enclosed:  # bench.py's phase markers: keep exactly the timed launches
            runs = enclosed
        runs = [(k, v) for k, v in runs if len(v) >= 5 and
                (k[0].startswith(tuple(kernels)) if kernels else not k[0].startswith("__amd"))]
        for label, (k, v) in zip(labels, runs):
            out.setdefault(label, {})["kernel"] = "%s [%d workgroups]" % k
        for label, (k, v) in zip(labels, runs):
            tail = v[-last:]
            got = out.setdefault(label, {})
            for c in tail[0]:
                if c not in ("key", "kernel"):
                    got[c] = statistics.median(x[c] for x in tail if c in x)
    return out


def account_markdown(runs) -> str:
    """Where a wave's cycles go, from counter_runs over the passes: the SQ
    wave-cycle counters partition a wave's life into issuing (ACTIVE_INST_ANY),
    waiting to issue (WAIT_INST_ANY: a dependency or a busy unit, the matrix
    core included) and waiting on anything else (WAIT_ANY: s_waitcnt,
    barriers); the issuing share is split by instruction type."""
    out = ["| counter | " + " | ".join(runs) + " |", "|---|" + "---|" * len(runs)]
    rows = [("dispatch us (under counters)", lambda c: "%.1f" % c["us"])]
    for name, num in (("issuing (ACTIVE_INST_ANY)", "SQ_ACTIVE_INST_ANY"),
                      ("waiting to issue (WAIT_INST_ANY)", "SQ_WAIT_INST_ANY"),
                      ("waiting on s_waitcnt / barrier (WAIT_ANY)", "SQ_WAIT_ANY"),
                      ("  issuing scalar (ACTIVE_INST_SCA)", "SQ_ACTIVE_INST_SCA"),
                      ("  issuing vector ALU incl. MFMA (ACTIVE_INST_VALU)", "SQ_ACTIVE_INST_VALU"),
                      ("  issuing LDS (ACTIVE_INST_LDS)", "SQ_ACTIVE_INST_LDS"),
                      ("  issuing vector memory (ACTIVE_INST_VMEM)", "SQ_ACTIVE_INST_VMEM")):
        rows.append((name + ", % of wave cycles",
                     lambda c, n=num: "%.1f" % (100 * c[n] / c["SQ_WAVE_CYCLES"])))
    rows += [("MFMA busy cycles per SIMD", lambda c: "%.0f" % (c["SQ_VALU_MFMA_BUSY_CYCLES"] / NUM_SIMD)),
             ("cycles per wave (4 x SQ_WAVE_CYCLES / waves)",
              lambda c: "%.0f" % (4 * c["SQ_WAVE_CYCLES"] / c["SQ_WAVES"])),
             ("vector-memory latency, cycles (VmemLatency)", lambda c: "%.0f" % c["VmemLatency"]),
             ("LDS latency, cycles (LdsLatency)", lambda c: "%.0f" % c["LdsLatency"]),
             ("TA address FIFO full, cycles per CU", lambda c: "%.0f" % (c["SQ_VMEM_TA_ADDR_FIFO_FULL"] / 256)),
             ("TA command FIFO full, cycles per CU", lambda c: "%.0f" % (c["SQ_VMEM_TA_CMD_FIFO_FULL"] / 256)),
             ("LDS data FIFO full, cycles per CU", lambda c: "%.0f" % (c["SQ_LDS_DATA_FIFO_FULL"] / 256)),
             ("scalar instructions per wave", lambda c: "%.0f" % (c["SQ_INSTS_SALU"] / c["SQ_WAVES"])),
             ("vector ALU instructions per wave (MFMA included)", lambda c: "%.0f" % (c["SQ_INSTS_VALU"] / c["SQ_WAVES"])),
             ("MFMA instructions per wave", lambda c: "%.0f" % (c["SQ_INSTS_MFMA"] / c["SQ_WAVES"])),
             ("LDS instructions per wave", lambda c: "%.0f" % (c["SQ_INSTS_LDS"] / c["SQ_WAVES"])),
             ("vector-memory instructions per wave", lambda c: "%.0f" % (c["SQ_INSTS_VMEM"] / c["SQ_WAVES"]))]
    for name, fn in rows:
        cells = []
        for c in runs.values():
            try:
                cells.append(fn(c))
            except (KeyError, ZeroDivisionError):
                cells.append("-")
        out.append("| %s | %s |" % (name, " | ".join(cells)))
    return "\n".join(out)


def lds_probe_rows(path: str, strides, skip: int = 3):
    """Bank-conflict counters of the LDS probe (bench.py --probes): its
    dispatches come in one group per stride, in order, `skip` warm-up
    launches first; per stride, the medians over the rest of SQ_INSTS_LDS,
    SQ_LDS_IDX_ACTIVE and SQ_LDS_BANK_CONFLICT, and the extra LDS cycles
    per conflict-free one, conflict / (active - conflict)."""
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    disp, order = {}, []
    for r in rows:
        if not short_name(r["Kernel_Name"]).startswith("lds_probe"):
            continue
        d = r.get("Dispatch_Id") or r["Start_Timestamp"]
        if d not in disp:
            disp[d] = {"us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3}
            order.append(d)
        disp[d][r["Counter_Name"]] = disp[d].get(r["Counter_Name"], 0.0) + float(
            r["Counter_Value"])
    per = len(order) // max(len(strides), 1)
    out = []
    for i, st in enumerate(strides):
        group = [disp[d] for d in order[i * per:(i + 1) * per]][skip:]
        med = {k: statistics.median(x[k] for x in group if k in x) for k in group[0]}
        act, conf = med.get("SQ_LDS_IDX_ACTIVE", 0.0), med.get("SQ_LDS_BANK_CONFLICT", 0.0)
        med["stride"] = st
        med["extra_per_cycle"] = conf / (act - conf) if act > conf else float("nan")
        out.append(med)
    return out


def mfma_markdown(rows) -> str:
    out = ["| kernel | us (under counters) | MFMA GFLOP counted | MFMA busy cycles per SIMD | "
           "wave cycles waiting (any) | wave cycles waiting (LDS) |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append("| %s | %.1f | %.1f | %.0f | %.1f %% | %.1f %% |" % (
            r["kernel"], r["us"], r["mfma_gflop"], r["busy_per_simd"], 100 * r["wait_any"],
            100 * r["wait_lds"]))
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
    t.add_argument("--timed", action="store_true",
                   help="only the runs bench.py's phase markers enclose: its timed launches")
    t.add_argument("--gap-ms", type=float, default=0.0,
                   help="also end a run where the device sat idle longer than this")
    t.add_argument("--last", type=int, default=0,
                   help="report runs of at least N consecutive dispatches by their last N "
                   "(steady state)")
    m = sub.add_parser("mfma", help="matrix-core work and wave waits from a --pmc pass "
                       "with SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_*, SQ_WAVE_CYCLES, "
                       "SQ_WAIT_INST_ANY, SQ_WAIT_INST_LDS")
    m.add_argument("dir")
    m.add_argument("--last", type=int, default=0)
    a = sub.add_parser("account", help="where a wave's cycles go, from several --pmc passes "
                       "of the same bench command (one run per workload)")
    a.add_argument("dirs", nargs="+")
    a.add_argument("--labels", required=True, help="comma-separated workload names, in order")
    a.add_argument("--last", type=int, default=8)
    lp = sub.add_parser("lds-probe", help="bank-conflict counters of the LDS probe per stride")
    lp.add_argument("dir")
    lp.add_argument("--strides", default="1,2,4,8,16,32,64")
    lp.add_argument("--skip", type=int, default=3)
    c = sub.add_parser("counters", help="calibrated HBM bytes per dispatch")
    c.add_argument("--fetch", required=True, help="dir of the FETCH_SIZE run")
    c.add_argument("--write", required=True, help="dir of the WRITE_SIZE run")
    c.add_argument("--copy-fetch", required=True, help="dir of the copy probe's FETCH_SIZE run")
    c.add_argument("--copy-write", required=True, help="dir of the copy probe's WRITE_SIZE run")
    c.add_argument("--copy-mib", type=float, required=True)
    c.add_argument("--labels", default="", help="comma-separated workload names, in the order "
                   "the bench ran them: one row per workload run instead of per kernel")
    args = ap.parse_args()
    if args.cmd == "stats":
        print(stats_markdown(kernel_stats(_find(args.dir, "_kernel_stats.csv"))))
        return
    if args.cmd == "mfma":
        print(mfma_markdown(mfma_rows(_find(args.dir, "_counter_collection.csv"), args.last)))
        return
    if args.cmd == "lds-probe":
        rows = lds_probe_rows(_find(args.dir, "_counter_collection.csv"),
                              [int(x) for x in args.strides.split(",")], args.skip)
        print("| lanes of a wave on one bank (stride) | us per launch (under counters) | "
              "LDS instructions | LDS busy cycles | bank-conflict cycles | "
              "extra cycles per conflict-free cycle |")
        print("|---|---|---|---|---|---|")
        for r in rows:
            print("| %d | %.1f | %.3g | %.4g | %.4g | %.2f |" % (
                r["stride"], r["us"], r.get("SQ_INSTS_LDS", float("nan")),
                r.get("SQ_LDS_IDX_ACTIVE", float("nan")), r.get("SQ_LDS_BANK_CONFLICT", float("nan")),
                r["extra_per_cycle"]))
        return
    if args.cmd == "account":
        runs = counter_runs([_find(d, "_counter_collection.csv") for d in args.dirs],
                            args.labels.split(","), args.last)
        print(account_markdown(runs))
        return
    if args.cmd == "trace":
        print(stats_markdown(dispatch_stats(_find(args.dir, "_kernel_trace.csv"), args.last,
                                            args.gap_ms, args.timed)))
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
    if args.labels:
        labels = args.labels.split(",")
        fr = counter_runs([_find(args.fetch, "_counter_collection.csv")], labels, 8, None)
        wr = counter_runs([_find(args.write, "_counter_collection.csv")], labels, 8, None)
        for lab in labels:
            if lab not in fr or lab not in wr:
                continue
            fb = fr[lab]["FETCH_SIZE"] * 1024 * f_fac
            wb = wr[lab]["WRITE_SIZE"] * 1024 * w_fac
            kern = fr[lab].get("kernel", "")
            print("%s, %s: fetch %.1f MB, write %.1f MB, total %.1f MB per dispatch (source %s)"
                  % (lab, kern, fb / 1e6, wb / 1e6, (fb + wb) / 1e6,
                     source_hash(kern.split("<")[0])))
        return
    for (k, n), v in sorted(fetch.items()):
        w = write.get((k, "WRITE_SIZE"), float("nan"))
        fb, wb = v * 1024 * f_fac, w * 1024 * w_fac
        print("%s: fetch %.1f MB, write %.1f MB, total %.1f MB per dispatch (source %s)"
              % (k, fb / 1e6, wb / 1e6, (fb + wb) / 1e6, source_hash(k.split("<")[0])))


if __name__ == "__main__":
    main()
