"""Summarise rocprofv3 output of bench.py into profiles/ (text + counter JSON).

This is the evidence generator for profiles/: every summary there names the
rocprofv3 command it was made from and the call of this script that wrote it.

Usage:
  python profile_summary.py trace  <kernel_stats.csv> <out.md> "<command>" [<dispatches.json>]
  python profile_summary.py dispatches <kernel_trace.csv> <kernel-substring> <source-key>
        <skip> <count> <bench_json_line_file> <stage> <out.json> "<command>"
  python profile_summary.py mfma <mfma_counter_collection.csv> <out.md> "<command>"
        <kernel-substring>@<grid>@<label>@<algorithmic flops> ...
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


def trace(stats_csv: str, out_md: str, command: str, dispatches_json: str | None = None):
    rows = _rows(stats_csv)
    lines = [f"# rocprofv3 kernel trace summary", "", f"Command: `{command}`", "",
             f"Written by: `python profile_summary.py trace <out>/trace_kernel_stats.csv {out_md} "
             f"\"<command>\"" + (f" {dispatches_json}`" if dispatches_json else "`"), ""]
    if dispatches_json:
        d = json.load(open(dispatches_json))
        lines += [f"The dominant kernel over the main step's eager timed loop (its dispatches "
                  f"{d['selected'][0] + 1} to {d['selected'][1]} in start order, the launches the "
                  f"HIP events time): average {d['trace_avg_us']:.1f} us (min "
                  f"{d['trace_min_us']:.1f}, max {d['trace_max_us']:.1f}); HIP events of the same "
                  f"run {d['events_same_run_us']:.1f} us. The table's average over all "
                  f"{d['dispatches_in_trace']} dispatches ({d['trace_all_dispatches_avg_us']:.1f} us) "
                  f"also holds the warm-up steps, the graph replays and the other legs' launches.", ""]
    lines += ["| kernel | calls | avg (us) | min (us) | max (us) | share |",
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


def dispatches(trace_csv, sub, source_key, skip, count, bench_json, stage, out_json, command):
    """Duration of the named kernel's dispatches number skip .. skip + count - 1 (in start
    order) of a rocprofv3 kernel trace: for bench.py's main step with --warmup W and
    --steps K, skip = W and count = K select exactly the eager timed loop's launches.
    Records their average next to the HIP-event average of the same stage printed by the
    same (traced) run, and the sha1 of the kernel's sources."""
    skip, count = int(skip), int(count)
    rows = [r for r in _rows(trace_csv) if sub in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    sel = us[skip:skip + count]
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    rec = {"kernel": sub, "source_key": source_key, "dispatches_in_trace": len(us),
           "selected": [skip, skip + count], "dispatches": len(sel),
           "trace_avg_us": statistics.mean(sel), "trace_min_us": min(sel),
           "trace_max_us": max(sel), "trace_all_dispatches_avg_us": statistics.mean(us),
           "events_same_run_us": line["kernels"][stage]["ms"] * 1e3,
           "kernel_sources_sha1": bench.kernel_source_hash(source_key), "command": command}
    json.dump(rec, open(out_json, "w"), indent=1)
    print(json.dumps(rec))


def mfma(csv_path, out_md, command, *kernels):
    """MfmaUtil and MfmaFlopsBF16 (rocprofv3 derived counters) averaged per launch of each
    named kernel of the given grid size (work-items), next to its algorithmic flops."""
    rows = _rows(csv_path)
    lines = ["# MFMA utilisation (rocprofv3 derived counters)", "", f"Command: `{command}`", "",
             "`MfmaUtil` = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMDs);",
             "`MfmaFlopsBF16` = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (flops the matrix cores executed).",
             "", "| kernel | workload | launches | MfmaUtil | MFMA flops executed | algorithmic flops |",
             "|---|---|---|---|---|---|"]
    for spec in kernels:
        sub, grid, label, algo = spec.split("@")
        vals = {"MfmaUtil": [], "MfmaFlopsBF16": []}
        for r in rows:
            if sub in r["Kernel_Name"] and r["Grid_Size"] == grid and r["Counter_Name"] in vals:
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
        n = len(vals["MfmaUtil"])
        lines.append(f"| `{sub}` | {label} | {n} | {statistics.mean(vals['MfmaUtil']):.1f} % | "
                     f"{statistics.mean(vals['MfmaFlopsBF16']) / 1e9:.2f} G | {float(algo) / 1e9:.2f} G |")
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
    rec = {"kernel": sub, "source_key": source_key, "grid_size": grid, "first": first,
           "launches": len(f), "fetch_kib_raw": statistics.mean(f),
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
        trace(*sys.argv[2:6])
    elif sys.argv[1] == "dispatches":
        dispatches(*sys.argv[2:11])
    elif sys.argv[1] == "mfma":
        mfma(*sys.argv[2:])
    else:
        counters(*sys.argv[2:9], *sys.argv[9:])
