"""Turn rocprofv3 CSV output into the per-kernel summaries kept under profiles/.

    python -m log_linear_attention_attn_amd.profiling stats  <kernel_stats.csv>  [--title T] [--command C]
    python -m log_linear_attention_attn_amd.profiling trace  <kernel_trace.csv>
    python -m log_linear_attention_attn_amd.profiling traffic --fetch <dir> --write <dir>
           --copy-fetch <dir> --copy-write <dir> --copy-bytes N --kernel NAME --workload W --command C

The traffic mode reads two --pmc runs of the workload (FETCH_SIZE, WRITE_SIZE,
KiB per dispatch) and two of a plain device copy of a known byte count.  The
counters are scaled by (known copy bytes / what they report for the copy), so
the recorded HBM traffic per launch is in true bytes.  The record carries the
hash of the kernel sources; bench.py reports it only while the sources match.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "log_linear_attention_attn_amd", "csrc")
HASHED = ("loglinear_fwd.hip", "loglinear_sweep_rs.hip", "loglinear_sweep_wide.hip", "ll_device.h",
          "ll_internal.h", "loglinear_api.cpp")


def source_hash() -> str:
    h = hashlib.sha256()
    for f in HASHED:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def counter_per_dispatch(d: str, kernel_substr: str, counter: str) -> float:
    vals = [float(r["Counter_Value"]) for r in _counter_rows(d)
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise ValueError(f"no {counter} rows for '{kernel_substr}' under {d}")
    return statistics.median(vals)


def traffic(args) -> dict:
    fetch_kib = counter_per_dispatch(args.fetch, args.kernel, "FETCH_SIZE")
    write_kib = counter_per_dispatch(args.write, args.kernel, "WRITE_SIZE")
    cf = counter_per_dispatch(args.copy_fetch, args.copy_kernel, "FETCH_SIZE")
    cw = counter_per_dispatch(args.copy_write, args.copy_kernel, "WRITE_SIZE")
    f_scale = args.copy_bytes / (cf * 1024.0)
    w_scale = args.copy_bytes / (cw * 1024.0)
    read_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    return {
        "kernel": args.kernel, "workload": args.workload, "source_hash": source_hash(),
        "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
        "copy_bytes": args.copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "read_bytes_per_launch": read_b, "write_bytes_per_launch": write_b,
        "bytes_per_launch": read_b + write_b, "command": args.command,
    }


def stats(path: str) -> list[dict]:
    with open(path) as fh:
        rows = list(csv.DictReader(fh))
    out = []
    for r in rows:
        out.append({"name": r.get("Name") or r.get("KERNEL_NAME") or r.get("Kernel_Name"),
                    "calls": int(float(r.get("Calls", 0))),
                    "total_ns": float(r.get("TotalDurationNs", 0)),
                    "avg_ns": float(r.get("AverageNs", 0)),
                    "pct": float(r.get("Percentage", 0))})
    return out


def trace(path: str, context: str | None = None) -> list[dict]:
    """Per (kernel, grid size) dispatch count and mean / median duration from
    a rocprofv3 kernel_trace.csv: one bench run times several workloads with
    the same kernels, and the grid tells their launches apart.  With context
    (a kernel-name substring), dispatches are further keyed by the grid of the
    latest dispatch of that kernel before them (e.g. the segment-state kernel,
    whose grid differs between the workloads a sweep kernel serves)."""
    groups: dict[tuple, list[float]] = {}
    with open(path) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))
    ctx = 0
    for r in rows:
        gx = int(r["Grid_Size_X"])
        if context and context in r["Kernel_Name"]:
            ctx = gx
        key = (r["Kernel_Name"], gx, int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]), ctx if context else 0)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = []
    for (name, gx, gy, gz, wx, cg), d in groups.items():
        out.append({"name": name, "grid": (gx, gy, gz), "block": wx, "context_grid": cg, "calls": len(d),
                    "mean_us": statistics.fmean(d), "median_us": statistics.median(d), "total_us": sum(d)})
    out.sort(key=lambda r: -r["total_us"])
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    tr.add_argument("--context")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write", "kernel", "workload", "command"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--out")
    args = ap.parse_args(argv)
    if args.mode == "trace":
        for r in trace(args.csv, args.context):
            g = "x".join(str(v) for v in r["grid"])
            c = f" after {args.context} grid {r['context_grid']}" if args.context else ""
            print(f"{r['calls']:6d}  mean {r['mean_us']:9.2f} us  median {r['median_us']:9.2f} us  "
                  f"grid {g:>16s} block {r['block']:4d}  {r['name'][:80]}{c}")
    elif args.mode == "stats":
        for r in stats(args.csv):
            print(f"{r['calls']:6d}  {r['avg_ns'] / 1e3:10.2f} us  {r['pct']:6.2f}%  {r['name'][:110]}")
    else:
        rec = traffic(args)
        js = json.dumps(rec, indent=1)
        if args.out:
            with open(args.out, "w") as fh:
                fh.write(js + "\n")
        print(js)


if __name__ == "__main__":
    sys.exit(main())
