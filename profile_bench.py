#!/usr/bin/env python3
"""Turns rocprofv3 CSV output of bench.py runs into the short summaries kept
under profiles/.

  kernels  STATS_CSV OUT_MD "COMMAND"
      per-kernel calls / average / min / max duration from a
      `rocprofv3 --kernel-trace --stats -f csv` run (the *_kernel_stats.csv).

  traffic  FETCH_CSV WRITE_CSV CALIB_MIB OUT_JSON "COMMAND" "COMMAND"
      HBM bytes per dispatch of every kernel from two
      `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE -f csv` runs (the
      *_counter_collection.csv files) of `bench.py --calib CALIB_MIB`.
      FETCH_SIZE and WRITE_SIZE count KiB; FETCH_SIZE is scaled by the factor
      that makes this project's streaming read probe (k_probe_read) of
      CALIB_MIB MiB read exactly that, WRITE_SIZE by the factor that makes
      the streaming write probe (k_probe_write) write exactly that.  The JSON
      carries bench.source_hash() so bench.py ignores it once the kernel
      sources change.

  counters COUNTER_CSV OUT_MD "COMMAND" KERNEL [KERNEL...]
      per-dispatch averages of every counter in a `rocprofv3 --pmc ...`
      run, for the named kernels (short names; a prefix matches).
"""
from __future__ import annotations

import csv
import json
import os
import statistics
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

READ_PROBE = "k_probe_read"
WRITE_PROBE = "k_probe_write"


def short_name(name: str) -> str:
    """Kernel name without the anonymous namespace and parameter list."""
    n = name.replace("(anonymous namespace)::", "").strip()
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def kernels(stats_csv: str, out_md: str, command: str) -> None:
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    lines = ["# Kernel durations (rocprofv3 --kernel-trace --stats)", "",
             "Command (run from the repository root, one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | average us | min us | max us | share |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} % |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_dispatch(counter_csv: str, counter: str) -> dict:
    """kernel short name -> list of per-dispatch counter values."""
    out = defaultdict(list)
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                out[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def traffic(fetch_csv: str, write_csv: str, calib_mib: int, out_json: str, cmd_fetch: str,
            cmd_write: str) -> None:
    import bench
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    known_kib = calib_mib * 1024.0
    f_probe = statistics.mean(fetch[READ_PROBE])
    w_probe = statistics.mean(write[WRITE_PROBE])
    f_scale, w_scale = known_kib / f_probe, known_kib / w_probe
    res = {"source_hash": bench.source_hash(),
           "counters": "FETCH_SIZE and WRITE_SIZE (KiB per dispatch), averaged over dispatches",
           "calibration": {"read_kernel": READ_PROBE, "write_kernel": WRITE_PROBE,
                           "bytes": calib_mib << 20, "fetch_kib": f_probe, "write_kib": w_probe,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "commands": [cmd_fetch, cmd_write], "kernels": {}}
    for name in sorted(set(fetch) & set(write)):
        if name in (READ_PROBE, WRITE_PROBE):
            continue
        fb = statistics.mean(fetch[name]) * 1024 * f_scale
        wb = statistics.mean(write[name]) * 1024 * w_scale
        res["kernels"][name] = {"dispatches": len(fetch[name]), "fetch_bytes": round(fb),
                                "write_bytes": round(wb)}
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


def counters(counter_csv: str, out_md: str, command: str, kernels_wanted) -> None:
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)  # kernel -> dispatch id -> duration in us (under the counter run)
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            name = short_name(r["Kernel_Name"])
            if any(name.startswith(k) for k in kernels_wanted):
                vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                    durs[name][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    names = sorted({c for v in vals.values() for c in v})
    lines = ["# Counters per dispatch (rocprofv3 --pmc)", "", "Command (run from the repository root, one MI355X):",
             "", "```", command, "```", "",
             "`us` is the average dispatch duration in the counter run itself.", "",
             "| kernel | dispatches | us | " + " | ".join(names) + " |",
             "|---|---:|---:|" + "---:|" * len(names)]
    for k in sorted(vals):
        n = max(len(v) for v in vals[k].values())
        us = f"{statistics.mean(durs[k].values()):.2f}" if durs.get(k) else ""
        cells = [f"{statistics.mean(vals[k][c]):.4g}" if vals[k].get(c) else "" for c in names]
        lines.append(f"| `{k}` | {n} | {us} | " + " | ".join(cells) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "kernels":
        kernels(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 8 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6], sys.argv[7])
    elif len(sys.argv) >= 6 and sys.argv[1] == "counters":
        counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    else:
        print(__doc__, file=sys.stderr)
        sys.exit(2)
