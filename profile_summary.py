#!/usr/bin/env python3
"""Summarise rocprofv3 CSV output into the short text files kept under ``profiles/``.

  trace    per (kernel, grid size): calls, average / min / max duration, from a
           ``*_kernel_trace.csv`` of ``rocprofv3 --kernel-trace --stats``. Workloads that
           launch the same kernel with the same grid are told apart by run order with
           ``--split KERNEL@GRID=label1,label2,...``: consecutive runs of that kernel and grid
           (in dispatch order, a run ending where another kernel is dispatched) get the labels
           in turn, the last label taking every later run.
  traffic  HBM bytes per launch of one kernel from two ``--pmc`` runs (FETCH_SIZE, then
           WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a
           plain copy kernel of known size run in the same process (the Ulysses permute:
           every call reads and writes the same known number of bytes). Writes the JSON
           that bench.py reports as ``roofline.traffic`` (only while the kernel source hash
           still matches). ``--first N`` keeps the kernel's first N dispatches only (the
           headline runs first in bench.py; later workloads may share its grid size).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import statistics


def _short(name: str) -> str:
    name = name.replace("ra::(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "").strip()


def trace(args):
    splits = {}
    for spec in args.split:
        key, labels = spec.split("=", 1)
        kern, grid = key.rsplit("@", 1)
        splits[(kern, int(grid))] = labels.split(",")
    rows = sorted(csv.DictReader(open(args.csv)), key=lambda r: int(r["Dispatch_Id"]))
    groups = collections.defaultdict(list)
    run_no = collections.Counter()
    prev = None
    for r in rows:
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]))
        label = ""
        if key in splits:
            if key != prev:
                run_no[key] += 1
            names = splits[key]
            label = names[min(run_no[key], len(names)) - 1]
        prev = key
        groups[key + (label,)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    lines = [f"# {args.title}", "", f"Command: `{args.cmd}`", "",
             "| kernel | grid (threads) | workload | calls | avg ms | min ms | max ms |",
             "|---|---|---|---|---|---|---|"]
    for (k, g, lab), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {k} | {g} | {lab} | {len(v)} | {statistics.mean(v):.4f} | {min(v):.4f} | {max(v):.4f} |")
    text = "\n".join(lines) + "\n"
    if args.note:
        text += "\n" + args.note + "\n"
    open(args.out, "w").write(text)
    print(text)


def _counter(path, kernel, grid, name, first=0):
    rows = [r for r in csv.DictReader(open(path))
            if _short(r["Kernel_Name"]).startswith(kernel) and int(r["Grid_Size"]) == grid
            and r["Counter_Name"] == name]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    vals = [float(r["Counter_Value"]) for r in rows][: first or None]
    if not vals:
        raise SystemExit(f"no {name} samples for {kernel} grid {grid} in {path}")
    return statistics.mean(vals), len(vals)


def traffic(args):
    f_k, nf = _counter(args.fetch, args.kernel, args.grid, "FETCH_SIZE", args.first)
    w_k, nw = _counter(args.write, args.kernel, args.grid, "WRITE_SIZE", args.first)
    f_c, _ = _counter(args.fetch, args.calib_kernel, args.calib_grid, "FETCH_SIZE")
    w_c, _ = _counter(args.write, args.calib_kernel, args.calib_grid, "WRITE_SIZE")
    ff = args.calib_bytes / (f_c * 1024.0)
    fw = args.calib_bytes / (w_c * 1024.0)
    fetch_b = f_k * 1024.0 * ff
    write_b = w_k * 1024.0 * fw
    src_hash = hashlib.sha256(open(args.src, "rb").read()).hexdigest()[:16]
    out = {"kernel": args.kernel, "grid": args.grid, "bytes_per_launch": round(fetch_b + write_b),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "fetch_kib_raw": f_k, "write_kib_raw": w_k, "launches": [nf, nw],
           "calibration": {"kernel": args.calib_kernel, "grid": args.calib_grid, "bytes_each_way": args.calib_bytes,
                           "fetch_kib_raw": f_c, "write_kib_raw": w_c, "fetch_factor": ff, "write_factor": fw},
           "kernel_sha256_16": src_hash, "commands": args.cmd}
    json.dump(out, open(args.out, "w"), indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--out", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--note", default="")
    t.add_argument("--split", action="append", default=[])
    w = sub.add_parser("traffic")
    w.add_argument("--fetch", required=True)
    w.add_argument("--write", required=True)
    w.add_argument("--kernel", required=True)
    w.add_argument("--grid", type=int, required=True)
    w.add_argument("--first", type=int, default=0)
    w.add_argument("--calib-kernel", required=True)
    w.add_argument("--calib-grid", type=int, required=True)
    w.add_argument("--calib-bytes", type=int, required=True)
    w.add_argument("--src", required=True)
    w.add_argument("--cmd", required=True)
    w.add_argument("--out", required=True)
    args = ap.parse_args()
    (trace if args.mode == "trace" else traffic)(args)


if __name__ == "__main__":
    main()
