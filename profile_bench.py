#!/usr/bin/env python3
"""Turns rocprofv3 CSV output of bench.py runs into the short summaries kept
under profiles/.

  kernels  STATS_CSV OUT_MD "COMMAND"
      per-kernel calls / average / min / max duration from a
      `rocprofv3 --kernel-trace --stats -f csv` run (the *_kernel_stats.csv).

  traffic  FETCH_CSV WRITE_CSV COPY_MIB OUT_JSON "COMMAND" "COMMAND"
      HBM bytes per dispatch of every kernel from two
      `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE -f csv` runs (the
      *_counter_collection.csv files) of `bench.py --calib-copy COPY_MIB`.
      FETCH_SIZE and WRITE_SIZE count KiB; each is scaled by the factor that
      makes the plain device copy of COPY_MIB MiB (kernel
      __amd_rocclr_copyBuffer) read and write exactly COPY_MIB MiB.  The JSON
      carries bench.source_hash() so bench.py ignores it once the kernel
      sources change.
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

COPY_KERNEL = "__amd_rocclr_copyBuffer"


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
    """kernel short name -> list of per-dispatch counter values.  For the
    copy kernel only the dispatches with the largest grid are kept: those are
    the calibration copy (the runtime uses the same kernel for small copies
    of its own)."""
    out = defaultdict(list)
    copy_rows = []
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            name = short_name(r["Kernel_Name"])
            if name == COPY_KERNEL:
                copy_rows.append((int(r["Grid_Size"]), float(r["Counter_Value"])))
            else:
                out[name].append(float(r["Counter_Value"]))
    if copy_rows:
        g = max(c[0] for c in copy_rows)
        out[COPY_KERNEL] = [v for gs, v in copy_rows if gs == g]
    return out


def traffic(fetch_csv: str, write_csv: str, copy_mib: int, out_json: str, cmd_fetch: str,
            cmd_write: str) -> None:
    import bench
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    known_kib = copy_mib * 1024.0
    f_copy = statistics.mean(fetch[COPY_KERNEL])
    w_copy = statistics.mean(write[COPY_KERNEL])
    f_scale, w_scale = known_kib / f_copy, known_kib / w_copy
    res = {"source_hash": bench.source_hash(),
           "counters": "FETCH_SIZE and WRITE_SIZE (KiB per dispatch), averaged over dispatches",
           "calibration": {"kernel": COPY_KERNEL, "bytes": copy_mib << 20,
                           "fetch_kib": f_copy, "write_kib": w_copy,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "commands": [cmd_fetch, cmd_write], "kernels": {}}
    for name in sorted(set(fetch) & set(write)):
        if name == COPY_KERNEL:
            continue
        fb = statistics.mean(fetch[name]) * 1024 * f_scale
        wb = statistics.mean(write[name]) * 1024 * w_scale
        res["kernels"][name] = {"dispatches": len(fetch[name]), "fetch_bytes": round(fb),
                                "write_bytes": round(wb)}
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "kernels":
        kernels(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 8 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5], sys.argv[6], sys.argv[7])
    else:
        print(__doc__, file=sys.stderr)
        sys.exit(2)
