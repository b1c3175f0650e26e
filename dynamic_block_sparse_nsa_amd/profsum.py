"""Summaries of rocprofv3 output for the benchmark's profile records.

``stats``   kernel_trace.csv (from ``rocprofv3 --kernel-trace -f csv``) -> a short text table
            of calls, average and total duration per kernel and launch size (workgroups),
            so launches of one kernel on different workloads get rows of their own.
``counters`` counter_collection.csv files of several --pmc passes -> per-kernel table of
            every counter and derived metric (MFMA busy, VALU busy, LDS use, L2 hits, ...).
``traffic`` two counter_collection.csv files (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``)
            -> HBM bytes per launch of each named kernel (its largest launch, the headline
            workload), scaled by what the same counter reads for a plain device copy of
            known size in the same run, written into a
            JSON record with the hash of the kernel's sources (a record whose hash no
            longer matches the sources is ignored by the benchmark).

Usage:
  python -m dynamic_block_sparse_nsa_amd.profsum stats TRACE_CSV --cmd "..." --title "..." > out.txt
  python -m dynamic_block_sparse_nsa_amd.profsum traffic --fetch F.csv --write W.csv \
      --copy-bytes N --copy-regex REGEX --kernel NAME=SRC[,SRC...] [--kernel ...] --out traffic.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def source_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    if name.startswith(("void at::", "at::")):
        return "(torch kernel: input generation / copy)"
    name = name.replace("(anonymous namespace)::", "")
    m = re.match(r"(?:void )?(?:nsa::)?([A-Za-z_0-9]+)(<[^()]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name


def stats(path: str, cmd: str, title: str) -> str:
    groups = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups[(short_name(r["Kernel_Name"]), grid // max(wg, 1))].append(dur)
    total = sum(sum(v) for v in groups.values())
    rows = sorted(((n, w, len(v), sum(v) / len(v), sum(v)) for (n, w), v in groups.items()), key=lambda r: -r[4])
    out = [f"# {title}", "", f"command: {cmd}", "",
           f"{'kernel':52s} {'wgs':>8s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s} {'pct':>6s}"]
    for name, wgs, calls, avg, tot in rows:
        out.append(f"{name[:52]:52s} {wgs:8d} {calls:6d} {avg:10.1f} {tot / 1e3:10.2f} {100 * tot / total:6.2f}")
    return "\n".join(out) + "\n"


def per_kernel_counter(path: str, counter: str) -> dict:
    """Mean of a counter's per-dispatch value per kernel name, over that kernel's largest
    launches (the headline workload when one kernel also runs on smaller ones)."""
    acc = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc[r["Kernel_Name"]][int(r["Grid_Size"])].append(float(r["Counter_Value"]))
    out = {}
    for k, by_grid in acc.items():
        v = by_grid[max(by_grid)]
        out[k] = sum(v) / len(v)
    return out


def pick(values: dict, regex: str) -> float:
    hits = [v for k, v in values.items() if re.search(regex, k)]
    if not hits:
        raise SystemExit(f"no kernel matches {regex!r} among {sorted(values)[:8]}")
    return max(hits)


def traffic(fetch_csv, write_csv, copy_bytes, copy_regex, kernels, out_path, cmd, util_csv=None):
    fetch = per_kernel_counter(fetch_csv, "FETCH_SIZE")
    write = per_kernel_counter(write_csv, "WRITE_SIZE")
    util = per_kernel_counter(util_csv, "MfmaUtil") if util_csv else {}
    # counters are in KiB per dispatch; the copy reads and writes copy_bytes exactly
    f_scale = copy_bytes / (pick(fetch, copy_regex) * 1024.0)
    w_scale = copy_bytes / (pick(write, copy_regex) * 1024.0)
    rec = json.load(open(out_path)) if os.path.exists(out_path) else {}
    for spec in kernels:
        name, srcs = spec.split("=", 1)
        srcs = srcs.split(",")
        fb = pick(fetch, rf"\b{re.escape(name)}\b") * 1024.0 * f_scale
        wb = pick(write, rf"\b{re.escape(name)}\b") * 1024.0 * w_scale
        rec[name] = {"fetch_bytes_per_launch": int(fb), "write_bytes_per_launch": int(wb),
                     "bytes_per_launch": int(fb + wb), "fetch_scale": round(f_scale, 4),
                     "write_scale": round(w_scale, 4), "copy_bytes": copy_bytes,
                     "sources": srcs, "source_sha": source_sha(srcs), "command": cmd}
        hits = [v for k, v in util.items() if re.search(rf"\b{re.escape(name)}\b", k)]
        if hits:   # fraction of the MFMA pipes' cycles busy (rocprofv3 MfmaUtil, same command)
            rec[name]["mfma_busy_frac"] = round(max(hits) / 100.0, 4)
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def counters(csvs, cmd: str, title: str, kernel_regex: str = "") -> str:
    """Per-kernel table of every counter found in the given counter_collection.csv files
    (several rocprofv3 --pmc passes of one command), each the mean over the kernel's largest
    launches.  Derived metrics (MfmaUtil, VALUBusy, LdsUtil, ...) are reported as rocprofv3
    computed them."""
    table = defaultdict(dict)
    names = []
    for path in csvs:
        acc = defaultdict(lambda: defaultdict(lambda: defaultdict(list)))
        with open(path) as f:
            for r in csv.DictReader(f):
                acc[r["Counter_Name"]][short_name(r["Kernel_Name"])][int(r["Grid_Size"])].append(
                    float(r["Counter_Value"]))
        for cname, per_k in acc.items():
            if cname not in names:
                names.append(cname)
            for k, by_grid in per_k.items():
                g = max(by_grid)
                v = by_grid[g]
                table[(k, g)][cname] = sum(v) / len(v)
    rows = sorted(table.items(), key=lambda kv: kv[0][0])
    out = [f"# {title}", "", f"command: {cmd}", "", "Each value: mean per dispatch over the kernel's largest launch "
           "(grid size in threads).", ""]
    for (k, g), vals in rows:
        if kernel_regex and not re.search(kernel_regex, k):
            continue
        out.append(f"{k}  (grid {g})")
        for c in names:
            if c in vals:
                v = vals[c]
                out.append(f"    {c:34s} {v:18.4f}" if abs(v) < 1e6 else f"    {c:34s} {v:18.0f}")
        out.append("")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--copy-regex", required=True)
    b.add_argument("--kernel", action="append", required=True)
    b.add_argument("--out", required=True)
    b.add_argument("--cmd", default="")
    b.add_argument("--util", default=None, help="counter CSV with MfmaUtil (optional)")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--kernels", default="")
    args = ap.parse_args(argv)
    if args.what == "stats":
        sys.stdout.write(stats(args.csv, args.cmd, args.title))
    elif args.what == "counters":
        sys.stdout.write(counters(args.csv, args.cmd, args.title, args.kernels))
    else:
        rec = traffic(args.fetch, args.write, args.copy_bytes, args.copy_regex, args.kernel, args.out, args.cmd,
                      args.util)
        print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
