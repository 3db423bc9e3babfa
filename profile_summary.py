"""Summarise rocprofv3 output of bench.py into profiles/ (text + counter JSON).

Usage:
  python profile_summary.py trace  <kernel_stats.csv> <out.md> "<command>"
  python profile_summary.py counters <fetch_counter_collection.csv> <write_counter_collection.csv>
        <kernel-substring> <source-key> <out.json> "<fetch command>" "<write command>"
        [grid=<work-items>] [first=<n>]

For a kernel that bench.py also launches in other legs, grid= keeps only the
dispatches of that grid size (work-items, as rocprofv3 reports it) and first=
only the first n of those in dispatch order (bench.py runs the main step
before the extended step and the ES-dLLM legs).

<source-key> names the kernel's source files in bench.KERNEL_SOURCES.

`counters` scales FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the named
kernel by the ratio of the known byte count of bench.py's calibration copy
(256 MiB, --copy-calibration) to what the same counter reads for that copy,
and records the sha1 of the kernel's sources, so that bench.py only reports
the traffic while the kernel is unchanged.
"""
from __future__ import annotations

import csv
import json
import statistics
import sys

import bench

COPY_KERNEL = "copyBuffer"


def _rows(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


def trace(stats_csv: str, out_md: str, command: str):
    rows = _rows(stats_csv)
    lines = [f"# rocprofv3 kernel trace summary", "", f"Command: `{command}`", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        short = name.split("(")[0]
        if short.startswith("void at::native") or short.startswith("at::native"):
            short = "torch input generation: " + short[:40] + "…"
        lines.append(f"| {short[:70]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _per_kernel(path, counter, sub, grid=None, first=None):
    """Counter values of the named kernel's dispatches (of grid size `grid` and
    the first `first` of them, if given), and of the calibration copy (the last
    copy dispatch with the largest grid: bench.py issues it last)."""
    vals, copies = [], []
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if sub in r["Kernel_Name"]:
            if grid is None or int(r["Grid_Size"]) == grid:
                vals.append((int(r["Dispatch_Id"]), v))
        elif COPY_KERNEL in r["Kernel_Name"]:
            copies.append((int(r["Grid_Size"]), int(r["Dispatch_Id"]), v))
    big = max(g for g, _, _ in copies)
    cal = [v for g, d, v in sorted(copies, key=lambda x: x[1]) if g == big][-1:]
    vals = [v for _, v in sorted(vals)]
    return (vals if first is None else vals[:first]), cal


def counters(fetch_csv, write_csv, sub, source_key, out_json, fetch_cmd, write_cmd, *select):
    opts = dict(a.split("=", 1) for a in select)
    grid = int(opts["grid"]) if "grid" in opts else None
    first = int(opts["first"]) if "first" in opts else None
    f, fcal = _per_kernel(fetch_csv, "FETCH_SIZE", sub, grid, first)
    w, wcal = _per_kernel(write_csv, "WRITE_SIZE", sub, grid, first)
    kib = 1024.0
    fscale = bench.COPY_CAL_BYTES / (max(fcal) * kib)
    wscale = bench.COPY_CAL_BYTES / (max(wcal) * kib)
    fetch = statistics.mean(f) * kib * fscale
    write = statistics.mean(w) * kib * wscale
    rec = {"kernel": sub, "grid_size": grid, "first": first, "launches": len(f), "fetch_kib_raw": statistics.mean(f),
           "write_kib_raw": statistics.mean(w), "copy_fetch_kib_raw": max(fcal),
           "copy_write_kib_raw": max(wcal), "copy_bytes": bench.COPY_CAL_BYTES,
           "fetch_scale": fscale, "write_scale": wscale,
           "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
           "traffic_bytes_per_launch": int(fetch + write),
           "kernel_sources_sha1": bench.kernel_source_hash(source_key),
           "commands": [fetch_cmd, write_cmd]}
    json.dump(rec, open(out_json, "w"), indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(*sys.argv[2:5])
    else:
        counters(*sys.argv[2:9], *sys.argv[9:])
