"""Summarise rocprofv3 CSV output of bench.py runs into profiles/.

Inputs (directories written by rocprofv3 -f csv -o bench):
  --trace DIR   --kernel-trace --stats run  (bench_kernel_stats.csv)
  --fetch DIR   --pmc FETCH_SIZE run        (bench_counter_collection.csv)
  --write DIR   --pmc WRITE_SIZE run        (bench_counter_collection.csv)

Counter calibration: the profiled bench runs a plain copy of known size
(`bench.py --calib`: torch.neg over 2^30 bytes of int32, reading and writing
2^30 bytes).  FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every kernel
are scaled by known / measured of that copy, giving bytes per launch.

Writes a markdown summary (--out) and, with --json, the per-kernel HBM bytes
per launch that bench.py reports as roofline.traffic, keyed by kernel and
tagged with the hash of the kernel sources they were measured on.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import sys

CALIB_BYTES = 1 << 30
CALIB_MATCH = "neg"


def _short(name: str) -> str:
    n = name.replace("unsigned int __vector(4)", "u32x4")
    return n if len(n) < 110 else n[:107] + "..."


def kernel_stats(d: str):
    rows = list(csv.DictReader(open(os.path.join(d, "bench_kernel_stats.csv"))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
             float(r["MaxNs"]), float(r["Percentage"])) for r in rows]


def counters(d: str, counter: str):
    rows = list(csv.DictReader(open(os.path.join(d, "bench_counter_collection.csv"))))
    agg = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]) * 1024.0)
    return {k: sum(v) / len(v) for k, v in agg.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--out", required=True)
    ap.add_argument("--json")
    ap.add_argument("--cmd", required=True, help="the bench command that was profiled")
    ap.add_argument("--title", default="bench.py")
    ap.add_argument("--workload", required=True, help="workload name the runs measured")
    args = ap.parse_args()

    ks = kernel_stats(args.trace)
    lines = [f"# rocprofv3 summary: {args.title}", "", "Command (kernel trace):", "",
             "```", f"rocprofv3 --kernel-trace --stats -f csv -d <dir> -o bench -- {args.cmd}", "```",
             "", "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in ks:
        lines.append(f"| `{_short(name)}` | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | "
                     f"{mx / 1e3:.1f} | {pct:.2f} |")
    traffic = {}
    if args.fetch and args.write:
        f = counters(args.fetch, "FETCH_SIZE")
        w = counters(args.write, "WRITE_SIZE")
        cal_f = [v for k, v in f.items() if CALIB_MATCH in k]
        cal_w = [v for k, v in w.items() if CALIB_MATCH in k]
        if not cal_f or not cal_w:
            sys.exit("calibration copy kernel not found in the counter runs")
        sf, sw = CALIB_BYTES / cal_f[0], CALIB_BYTES / cal_w[0]
        lines += ["", "Counters (separate runs, same bench with `--calib`):", "", "```",
                  f"rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o bench -- {args.cmd} --calib",
                  f"rocprofv3 --pmc WRITE_SIZE -f csv -d <dir> -o bench -- {args.cmd} --calib",
                  "```", "",
                  f"Calibration: a plain copy of 2^30 bytes reads FETCH_SIZE = {cal_f[0] / 1e9:.4f} GB "
                  f"and WRITE_SIZE = {cal_w[0] / 1e9:.4f} GB; scale factors {sf:.4f} (fetch), "
                  f"{sw:.4f} (write).", "",
                  "Values are per launch: the mean over the run's launches of each kernel. "
                  "bench.py reports the roofline kernel's scaled total as `traffic` "
                  "(from counters.json, while the kernel's code is unchanged).", "",
                  "| kernel | FETCH raw GB | WRITE raw GB | fetch GB (scaled) | write GB (scaled) | total GB |",
                  "|---|---|---|---|---|---|"]
        for k in sorted(set(f) & set(w), key=lambda k: -(f[k] + w[k])):
            if f[k] + w[k] < 1e6:
                continue
            fs, ws = f[k] * sf, w[k] * sw
            lines.append(f"| `{_short(k)}` | {f[k] / 1e9:.4f} | {w[k] / 1e9:.4f} | {fs / 1e9:.4f} | "
                         f"{ws / 1e9:.4f} | {(fs + ws) / 1e9:.4f} |")
            traffic[k] = fs + ws
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if args.json and traffic:
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        from bench import kernel_hash

        d = {}
        if os.path.exists(args.json):
            d = json.load(open(args.json))
        for k, v in traffic.items():
            for short in ("dispatch_copy", "combine_rows", "dispatch_fp8", "msg_pack_fp8",
                          "msg_pack_bf16", "msg_exec_puts", "msg_unpack"):
                if short in k:
                    d[f"{args.workload}:{short}"] = {"hbm_bytes_per_launch": round(v), "kernel": k,
                                                     "kernel_hash": kernel_hash(short),
                                                     "title": args.title}
        json.dump(d, open(args.json, "w"), indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    main()
