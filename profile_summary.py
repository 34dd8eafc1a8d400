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
           plain copy kernel of known size run in the same process (the HIP runtime's copy
           kernel behind the bench's 64 MiB device-to-device copy; median over its dispatches). Writes the JSON
           that bench.py reports as ``roofline.traffic`` (only while the kernel source hash
           still matches). ``--first N`` keeps the kernel's first N dispatches only (the
           headline runs first in bench.py; later workloads may share its grid size).
  pmc      per (kernel, grid) mean of every counter of one or more ``--pmc`` runs
           (``*_counter_collection.csv``), workloads told apart by run order as in ``trace``.
           ``MfmaUtil`` (rocprofiler's derived counter: matrix-core busy cycles over active
           cycles of every SIMD) is shown in percent; ``SQ_INSTS_VALU_MFMA_MOPS_BF16`` times 512
           is the bf16 matrix-core FLOP count each dispatch executed; with TCC_HIT_sum and
           TCC_MISS_sum the L2 hit rate is shown as well.
  hbm      HBM bandwidth of named kernels: mean duration from a kernel trace, algorithmic
           bytes per dispatch as given, and the bytes the counters saw (FETCH_SIZE and
           WRITE_SIZE runs, each scaled by what it reads for a plain device copy of known size
           in the same run: the HIP runtime's copy kernel behind a device-to-device copy).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import re
import statistics


def _demangle(name: str) -> str:
    """The tracer leaves some template instances mangled (those with a __bf16 parameter): turn
    ``_ZN<len><id>...<len><name>I<args>E...`` into ``name<args>`` for integer arguments."""
    if not name.startswith("_ZN"):
        return name
    i, ident = 3, ""
    while i < len(name) and name[i].isdigit():
        j = i
        while name[j].isdigit():
            j += 1
        n = int(name[i:j])
        ident, i = name[j:j + n], j + n
    args = []
    if name[i:i + 1] == "I":
        for m in re.finditer(r"Li(\d+)E", name[i + 1:]):
            args.append(m.group(1))
            if name[i + 1 + m.end():i + 2 + m.end()] == "E":
                break
    return ident + (f"<{', '.join(args)}>" if args else "") if ident else name


def _grid(r) -> int:
    """Threads of a dispatch: a kernel trace gives the grid per dimension, a counter run the total."""
    if "Grid_Size_X" in r:
        return int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
    return int(r["Grid_Size"])


def _short(name: str) -> str:
    name = _demangle(name).replace("ra::(anonymous namespace)::", "")
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
        key = (_short(r["Kernel_Name"]), _grid(r))
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
        # --last KERNEL@GRID=LABEL:N adds a row for the last N calls of that group (the timed
        # calls of a benchmark whose warm-up calls come first)
        for spec in args.last:
            key, rest = spec.split("=", 1)
            kern, grid = key.rsplit("@", 1)
            label, n = rest.rsplit(":", 1)
            if k == kern and g == int(grid) and lab == label:
                t = v[-int(n):]
                lines.append(f"| {k} | {g} | {lab}, last {len(t)} calls | {len(t)} | {statistics.mean(t):.4f} "
                             f"| {min(t):.4f} | {max(t):.4f} |")
    text = "\n".join(lines) + "\n"
    if args.note:
        text += "\n" + args.note + "\n"
    open(args.out, "w").write(text)
    print(text)


def _counter(path, kernel, grid, name, first=0, median=False):
    rows = [r for r in csv.DictReader(open(path))
            if _short(r["Kernel_Name"]).startswith(kernel) and int(r["Grid_Size"]) == grid
            and r["Counter_Name"] == name]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    vals = [float(r["Counter_Value"]) for r in rows][: first or None]
    if not vals:
        raise SystemExit(f"no {name} samples for {kernel} grid {grid} in {path}")
    return (statistics.median(vals) if median else statistics.mean(vals)), len(vals)


def traffic(args):
    f_k, nf = _counter(args.fetch, args.kernel, args.grid, "FETCH_SIZE", args.first)
    w_k, nw = _counter(args.write, args.kernel, args.grid, "WRITE_SIZE", args.first)
    # median: a runtime copy kernel of this grid may also serve other copies
    f_c, _ = _counter(args.fetch, args.calib_kernel, args.calib_grid, "FETCH_SIZE", median=True)
    w_c, _ = _counter(args.write, args.calib_kernel, args.calib_grid, "WRITE_SIZE", median=True)
    ff = args.calib_bytes / (f_c * 1024.0)
    fw = args.calib_bytes / (w_c * 1024.0)
    fetch_b = f_k * 1024.0 * ff
    write_b = w_k * 1024.0 * fw
    h = hashlib.sha256()
    for path in args.src:  # the kernel's source files, in the order bench.py hashes them
        h.update(open(path, "rb").read())
    src_hash = h.hexdigest()[:16]
    out = {"kernel": args.kernel, "grid": args.grid, "bytes_per_launch": round(fetch_b + write_b),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "fetch_kib_raw": f_k, "write_kib_raw": w_k, "launches": [nf, nw],
           "calibration": {"kernel": args.calib_kernel, "grid": args.calib_grid, "bytes_each_way": args.calib_bytes,
                           "fetch_kib_raw": f_c, "write_kib_raw": w_c, "fetch_factor": ff, "write_factor": fw},
           "kernel_sha256_16": src_hash, "commands": args.cmd}
    json.dump(out, open(args.out, "w"), indent=1)
    print(json.dumps(out, indent=1))


def _labelled(rows, splits, keyf):
    """Rows grouped by (kernel, grid, run-order label), in dispatch order."""
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    groups = collections.defaultdict(list)
    run_no = collections.Counter()
    prev = None
    for r in rows:
        key = keyf(r)
        label = ""
        if key in splits:
            if key != prev:
                run_no[key] += 1
            names = splits[key]
            label = names[min(run_no[key], len(names)) - 1]
        prev = key
        groups[key + (label,)].append(r)
    return groups


def _splits(specs):
    out = {}
    for spec in specs:
        key, labels = spec.split("=", 1)
        kern, grid = key.rsplit("@", 1)
        out[(kern, int(grid))] = labels.split(",")
    return out


def pmc(args):
    rows = []
    for path in args.csv:
        rows += list(csv.DictReader(open(path)))
    # one counter value per (dispatch, counter); a dispatch's counters share its Dispatch_Id
    per_disp = collections.defaultdict(dict)
    meta = {}
    for r in rows:
        d = (r.get("Agent_Id", ""), int(r["Dispatch_Id"]), r.get("_file", ""))
        per_disp[d][r["Counter_Name"]] = per_disp[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        meta[d] = r
    disp_rows = []
    for d, cnt in per_disp.items():
        m = dict(meta[d])
        m["_counters"] = cnt
        disp_rows.append(m)
    groups = _labelled(disp_rows, _splits(args.split), lambda r: (_short(r["Kernel_Name"]), int(r["Grid_Size"])))
    names = sorted({c for r in disp_rows for c in r["_counters"]})
    lines = [f"# {args.title}", "", f"Command: `{args.cmd}`", "",
             "| kernel | grid (threads) | workload | dispatches | " + " | ".join(names) +
             (" | bf16 MFMA TFLOP per dispatch" if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in names else "") +
             (" | L2 hit %" if {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(names) else "") + " |",
             "|---|---|---|---|" + "---|" * len(names) + ("---|" if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in names else "") +
             ("---|" if {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(names) else "")]
    for (k, g, lab), v in sorted(groups.items(), key=lambda kv: (kv[0][0], -kv[0][1], kv[0][2])):
        if args.kernel and not any(k.startswith(x) for x in args.kernel):
            continue
        cells = []
        for n in names:
            vals = [r["_counters"][n] for r in v if n in r["_counters"]]
            mean = statistics.mean(vals) if vals else float("nan")
            cells.append(f"{mean:.2f}" if n == "MfmaUtil" else f"{mean:.6g}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in names:
            mops = statistics.mean([r["_counters"]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for r in v])
            cells.append(f"{mops * 512 / 1e12:.4f}")
        if {"TCC_HIT_sum", "TCC_MISS_sum"} <= set(names):
            hit = sum(r["_counters"].get("TCC_HIT_sum", 0.0) for r in v)
            miss = sum(r["_counters"].get("TCC_MISS_sum", 0.0) for r in v)
            cells.append(f"{100 * hit / max(hit + miss, 1.0):.1f}")
        lines.append(f"| {k} | {g} | {lab} | {len(v)} | " + " | ".join(cells) + " |")
    text = "\n".join(lines) + "\n"
    if args.note:
        text += "\n" + args.note + "\n"
    open(args.out, "w").write(text)
    print(text)


def hbm(args):
    trace_rows = list(csv.DictReader(open(args.trace)))
    splits = _splits(args.split)
    tgroups = _labelled(trace_rows, splits, lambda r: (_short(r["Kernel_Name"]), _grid(r)))

    def counter_groups(path, name):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == name]
        return _labelled(rows, splits, lambda r: (_short(r["Kernel_Name"]), int(r["Grid_Size"])))

    fg = counter_groups(args.fetch, "FETCH_SIZE")
    wg = counter_groups(args.write, "WRITE_SIZE")

    def mean_of(groups, kern, grid, label, field):
        for (k, g, lab), v in groups.items():
            if k.startswith(kern) and g == grid and lab == label:
                return statistics.mean(float(r[field]) for r in v), len(v)
        raise SystemExit(f"no dispatches of {kern} grid {grid} label '{label}'")

    ck, cg = args.calib.split("=")[0].rsplit("@", 1)
    cbytes = int(args.calib.split("=")[1])
    def median_of(groups, kern, grid, field):
        # the runtime's copy kernel also serves other copies of this grid: take the median
        vals = [float(r[field]) for (k, g, _), v in groups.items() if k.startswith(kern) and g == grid for r in v]
        if not vals:
            raise SystemExit(f"no dispatches of {kern} grid {grid}")
        return statistics.median(vals)

    f_c = median_of(fg, ck, int(cg), "Counter_Value")
    w_c = median_of(wg, ck, int(cg), "Counter_Value")
    ff, fw = cbytes / (f_c * 1024.0), cbytes / (w_c * 1024.0)
    lines = [f"# {args.title}", "", f"Commands: `{args.cmd}`", "",
             f"Counter scale factors from the plain copy `{ck}` (grid {cg}, {cbytes} bytes each way): "
             f"FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f}.", "",
             "| kernel | grid (threads) | workload | avg ms | algorithmic bytes | algorithmic GB/s | % of 8 TB/s "
             "| counted read bytes | counted write bytes | counted / algorithmic |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for spec in args.kernel:
        key, rest = spec.split("=", 1)
        kern, grid = key.rsplit("@", 1)
        label, nbytes = rest.split(":")
        grid, nbytes = int(grid), int(nbytes)
        durs = None
        for (k, g, lab), v in tgroups.items():
            if k.startswith(kern) and g == grid and lab == label:
                durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in v]
        if not durs:
            raise SystemExit(f"no trace rows for {kern} grid {grid} label '{label}'")
        ms = statistics.mean(durs)
        f, _ = mean_of(fg, kern, grid, label, "Counter_Value")
        w, _ = mean_of(wg, kern, grid, label, "Counter_Value")
        rb, wb = f * 1024 * ff, w * 1024 * fw
        gbs = nbytes / (ms * 1e-3) / 1e9
        lines.append(f"| {kern} | {grid} | {label} | {ms:.4f} | {nbytes} | {gbs:.0f} | {100 * gbs / 8000:.1f} "
                     f"| {rb:.4g} | {wb:.4g} | {(rb + wb) / nbytes:.3f} |")
    text = "\n".join(lines) + "\n"
    if args.note:
        text += "\n" + args.note + "\n"
    open(args.out, "w").write(text)
    print(text)


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
    t.add_argument("--last", action="append", default=[], help="KERNEL@GRID=LABEL:N")
    w = sub.add_parser("traffic")
    w.add_argument("--fetch", required=True)
    w.add_argument("--write", required=True)
    w.add_argument("--kernel", required=True)
    w.add_argument("--grid", type=int, required=True)
    w.add_argument("--first", type=int, default=0)
    w.add_argument("--calib-kernel", required=True)
    w.add_argument("--calib-grid", type=int, required=True)
    w.add_argument("--calib-bytes", type=int, required=True)
    w.add_argument("--src", action="append", required=True)
    w.add_argument("--cmd", required=True)
    w.add_argument("--out", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("csv", nargs="+")
    p.add_argument("--out", required=True)
    p.add_argument("--title", required=True)
    p.add_argument("--cmd", required=True)
    p.add_argument("--note", default="")
    p.add_argument("--split", action="append", default=[])
    p.add_argument("--kernel", action="append", default=[], help="keep only kernels starting with this")
    h = sub.add_parser("hbm")
    h.add_argument("--trace", required=True)
    h.add_argument("--fetch", required=True)
    h.add_argument("--write", required=True)
    h.add_argument("--calib", required=True, help="KERNEL@GRID=BYTES_EACH_WAY of a plain copy")
    h.add_argument("--kernel", action="append", required=True, help="KERNEL@GRID=LABEL:ALGORITHMIC_BYTES")
    h.add_argument("--split", action="append", default=[])
    h.add_argument("--title", required=True)
    h.add_argument("--cmd", required=True)
    h.add_argument("--note", default="")
    h.add_argument("--out", required=True)
    args = ap.parse_args()
    {"trace": trace, "traffic": traffic, "pmc": pmc, "hbm": hbm}[args.mode](args)


if __name__ == "__main__":
    main()
