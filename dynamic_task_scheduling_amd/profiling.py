"""Summaries of rocprofv3 runs for profiles/ (text only; nothing here runs
on the GPU).

Every summary names the command that produced its input and the hash of the
kernel sources it was taken on (the same hash bench.py checks before it uses
a traffic figure).  Usage, from the repository root:

  python3 -m dynamic_task_scheduling_amd.profiling kernel-stats \\
      --csv OUT/run_kernel_stats.csv --workload NAME --command "..." --out profiles/X.md
  python3 -m dynamic_task_scheduling_amd.profiling traffic \\
      --fetch A.csv --write B.csv --copy-fetch C.csv --copy-write D.csv --copy-mib 1024 \\
      --workload NAME --kernel k_dynamic --algo-bytes N --command "..." ... --out profiles/Y.json
  python3 -m dynamic_task_scheduling_amd.profiling counters \\
      --csv OUT/run_counter_collection.csv --workload NAME --kernel k_dynamic \\
      --command "..." --out profiles/Z.md

Counter conventions on MI355X (checked against a plain device copy of known
size): FETCH_SIZE reads half the bytes a kernel fetches (it counts 64-byte
units for the 128-byte requests the L2 issues), WRITE_SIZE the full bytes;
both are in KiB per dispatch, summed over the XCDs.  SQ_* cycle counters are
summed over every SIMD (SQ_WAVE_CYCLES and the wait counters in units of 4
cycles), GRBM_GUI_ACTIVE over the 8 XCDs.
"""
import argparse
import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SIMDS = 256 * 4
XCDS = 8


def source_sha() -> str:
    sys.path.insert(0, ROOT)
    import bench
    return bench.kernel_source_sha()


def _short(name: str) -> str:
    n = name.replace("void ", "").split("(")[0]
    return n.replace("unsigned short", "bf16")


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def kernel_stats(args):
    rows = _rows(args.csv)
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = ["# %s on the %s workload: rocprofv3 kernel stats" % (args.kernel.rstrip("<"), args.workload), "",
           "Command (from the repository root, on one MI355X):", "", "    " + args.command, "",
           "Source hash of the kernels profiled: `%s` (sha256 of csrc/*.hip + *.hpp, first 16 hex)."
           % source_sha(), "",
           "| Kernel | Calls | Avg (us) | Min (us) | Max (us) | Share |", "|---|---|---|---|---|---|"]
    match = args.match.split(",")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        if not any(m in name for m in match):
            continue
        out.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f%% |" % (
            _short(name), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, 100.0 * float(r["TotalDurationNs"]) / total))
    if args.trace and args.timed:
        # per-dispatch durations of the kernel; the last `timed` dispatches
        # are the timed steps (the ones before them are warm-up)
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in _rows(args.trace)
             if args.kernel in r["Kernel_Name"]]
        t = sorted(d[-args.timed:])
        if t:
            med = t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])
            out += ["", "Timed dispatches of `%s` (the last %d of %d; the rest are warm-up): median %.1f us, "
                    "mean %.1f us, min %.1f us, max %.1f us." % (args.kernel.rstrip("<"), len(t), len(d), med,
                                                                  sum(t) / len(t), t[0], t[-1])]
    if args.note:
        out += ["", args.note]
    open(args.out, "w").write("\n".join(out) + "\n")


def _per_dispatch(path, counter, kernel):
    vals = defaultdict(float)
    for r in _rows(path):
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    return list(vals.values())


def traffic(args):
    f = _per_dispatch(args.fetch, "FETCH_SIZE", args.kernel)
    w = _per_dispatch(args.write, "WRITE_SIZE", args.kernel)
    cf = _per_dispatch(args.copy_fetch, "FETCH_SIZE", "copy")
    cw = _per_dispatch(args.copy_write, "WRITE_SIZE", "copy")
    cbytes = args.copy_mib * 1024 * 1024
    f_kib, w_kib = sum(f) / len(f), sum(w) / len(w)
    cf_kib, cw_kib = max(cf), max(cw)
    fs = cbytes / 1024.0 / cf_kib
    ws = cbytes / 1024.0 / cw_kib
    t = (f_kib * fs + w_kib * ws) * 1024.0
    d = {"workload": args.workload, "kernel": args.kernel.rstrip("<"), "source_sha": source_sha(),
         "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
         "dispatches": [len(f), len(w)],
         "copy_calibration": {"bytes": cbytes, "fetch_kib": cf_kib, "write_kib": cw_kib,
                              "fetch_scale": fs, "write_scale": ws},
         "traffic_bytes_per_launch": t, "algorithmic_bytes_per_launch": args.algo_bytes,
         "commands": args.command}
    json.dump(d, open(args.out, "w"), indent=1)


def counters(args):
    per = defaultdict(lambda: defaultdict(float))
    n = defaultdict(set)
    for r in _rows(args.csv):
        if args.kernel not in r["Kernel_Name"]:
            continue
        per[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
        n[r["Counter_Name"]].add(r["Dispatch_Id"])
    avg = {c: sum(v.values()) / len(v) for c, v in per.items()}
    out = ["# %s on the %s workload: rocprofv3 counters (per dispatch, averaged)" % (
        args.kernel.rstrip("<"), args.workload), "", "Command (from the repository root, on one MI355X):", "",
        "    " + args.command, "", "Source hash: `%s`." % source_sha(), "",
        "| Counter | Value |", "|---|---|"]
    for c in sorted(avg):
        out.append("| %s | %.4g |" % (c, avg[c]))
    g = avg.get("GRBM_GUI_ACTIVE")
    if g:
        cyc = g / XCDS
        out += ["", "Derived (cycles per XCD = GRBM_GUI_ACTIVE / 8 = %.4g):" % cyc, ""]
        if args.duration_us:
            out.append("* shader clock = cycles / kernel duration (%.1f us) = %.2f GHz" % (
                args.duration_us, cyc / (args.duration_us * 1e3)))
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            out.append("* MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles) = %.1f%%" % (
                100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / cyc))
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"):
            if c in avg:
                out.append("* %s = %.1f%% of wave-cycles (4 x value / (1024 waves x cycles))" % (
                    c, 100.0 * 4 * avg[c] / SIMDS / cyc))
        if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_LDS_IDX_ACTIVE" in avg and avg["SQ_LDS_IDX_ACTIVE"]:
            out.append("* LDS bank-conflict cycles / LDS active cycles = %.1f%%" % (
                100.0 * avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"]))
    if args.note:
        out += ["", args.note]
    open(args.out, "w").write("\n".join(out) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernel-stats")
    k.add_argument("--csv", required=True)
    k.add_argument("--workload", required=True)
    k.add_argument("--kernel", default="k_dynamic")
    k.add_argument("--command", required=True)
    k.add_argument("--note", default="")
    k.add_argument("--match", default="moe::,copyBuffer",
                   help="comma-separated substrings: kernels whose names hold one are listed")
    k.add_argument("--trace", default="", help="run_kernel_trace.csv of the same run")
    k.add_argument("--timed", type=int, default=0, help="timed dispatches at the end of the trace")
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--kernel", default="k_dynamic")
    t.add_argument("--algo-bytes", type=float, required=True)
    t.add_argument("--command", action="append", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--kernel", default="k_dynamic")
    c.add_argument("--command", required=True)
    c.add_argument("--duration-us", type=float, default=0.0)
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    {"kernel-stats": kernel_stats, "traffic": traffic, "counters": counters}[a.what](a)


if __name__ == "__main__":
    main()
