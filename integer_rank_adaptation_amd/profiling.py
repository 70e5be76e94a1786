"""Summaries of rocprofv3 output for the IntLoRA kernels (text in, text out).

    python -m integer_rank_adaptation_amd.profiling stats   --dir D --commands CMD...
    python -m integer_rank_adaptation_amd.profiling traffic --fetch D1 --write D2 \
        --copy-fetch D3 --copy-write D4 --copy-bytes B --workload NAME [--kernel k_linear]

`stats` reads the kernel trace of a `--kernel-trace --stats --output-format csv` run
and prints a markdown table (per kernel: calls, average and total duration, share of
GPU time) plus the per-launch durations of the linear layer grouped by grid size.

`traffic` reads the FETCH_SIZE and WRITE_SIZE counter runs (KiB per dispatch) of the
same command and of a plain device copy of known size, scales each counter by
copy bytes / counter reading of the copy, and prints JSON: HBM bytes per launch for
each kernel of the library, and the average over the launches of one kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OURS = re.compile(r"intlora::(k_\w+)(?:<([^>]*)>)?")


def kernel_source_sha():
    """Hash of the linear layer's sources; counter summaries record it so that a
    figure taken on another version of the kernel is not reused."""
    h = hashlib.sha256()
    for f in ("linear.hip", "device_common.h"):
        with open(os.path.join(ROOT, "integer_rank_adaptation_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(full):
    m = OURS.search(full)
    if m:
        return m.group(1) + (f"<{m.group(2)}>" if m.group(2) else "")
    s = re.sub(r"\(.*", "", full)
    return s[:60]


def _one(path, pattern):
    hits = sorted(glob.glob(os.path.join(path, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {path}")
    return hits[0]


def read_trace(d):
    rows = list(csv.DictReader(open(_one(d, "*kernel_trace.csv"))))
    out = []
    for r in rows:
        t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3  # us
        g = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
        out.append(dict(name=short_name(r["Kernel_Name"]), us=t, grid=g))
    return out


def stats(d, commands):
    tr = read_trace(d)
    total = sum(r["us"] for r in tr) or 1.0
    agg = collections.OrderedDict()
    for r in tr:
        a = agg.setdefault(r["name"], [0, 0.0])
        a[0] += 1
        a[1] += r["us"]
    lines = ["Commands (from the repository root, on one MI355X):", ""] + ["    " + c for c in commands] + ["",
             "| kernel | calls | avg us | total us | % of GPU time |", "|---|---:|---:|---:|---:|"]
    for name, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| `{name}` | {c} | {t / c:.2f} | {t:.1f} | {100 * t / total:.1f} |")
    lin = [r for r in tr if r["name"].startswith("k_linear")]
    if lin:
        by = collections.OrderedDict()
        for r in lin:
            by.setdefault((r["name"], r["grid"]), []).append(r["us"])
        lines += ["", "Linear layer launches by grid (threads):", "",
                  "| kernel | grid | launches | avg us | min us | max us |", "|---|---:|---:|---:|---:|---:|"]
        for (name, g), v in by.items():
            lines.append(f"| `{name}` | {g} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
        allv = [r["us"] for r in lin]
        lines += ["", f"All linear-layer launches: {len(allv)}, average {sum(allv) / len(allv):.2f} us."]
    return "\n".join(lines) + "\n"


def read_counter(d, counter):
    rows = list(csv.DictReader(open(_one(d, "*counter_collection.csv"))))
    out = []
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        out.append(dict(name=short_name(r["Kernel_Name"]), kib=float(r["Counter_Value"]),
                        grid=int(r.get("Grid_Size", 0) or 0), dispatch=int(r["Dispatch_Id"])))
    return out


def copy_factor(d, counter, nbytes):
    rows = read_counter(d, counter)
    big = max(rows, key=lambda r: r["kib"])  # the copy itself, not the set-up kernels
    return nbytes / (big["kib"] * 1024.0), big["kib"]


def traffic(fetch_dir, write_dir, cf_dir, cw_dir, copy_bytes, workload, kernel):
    ff, fk = copy_factor(cf_dir, "FETCH_SIZE", copy_bytes)
    wf, wk = copy_factor(cw_dir, "WRITE_SIZE", copy_bytes)
    fe = read_counter(fetch_dir, "FETCH_SIZE")
    wr = read_counter(write_dir, "WRITE_SIZE")
    per = collections.OrderedDict()
    for r in fe:
        if not r["name"].startswith("k_"):
            continue
        per.setdefault((r["name"], r["grid"]), dict(fetch=[], write=[]))["fetch"].append(r["kib"] * 1024 * ff)
    for r in wr:
        if not r["name"].startswith("k_"):
            continue
        per.setdefault((r["name"], r["grid"]), dict(fetch=[], write=[]))["write"].append(r["kib"] * 1024 * wf)
    kernels = []
    for (name, g), v in per.items():
        f = sum(v["fetch"]) / max(1, len(v["fetch"]))
        w = sum(v["write"]) / max(1, len(v["write"]))
        kernels.append(dict(kernel=name, grid=g, launches=len(v["fetch"]), fetch_bytes=round(f), write_bytes=round(w),
                            hbm_bytes=round(f + w)))
    sel = [k for k in kernels if k["kernel"].startswith(kernel)]
    nl = sum(k["launches"] for k in sel)
    avg = sum(k["hbm_bytes"] * k["launches"] for k in sel) / nl if nl else None  # per launch
    return dict(workload=workload, kernel=kernel, kernel_source_sha=kernel_source_sha(),
                copy_bytes=copy_bytes, copy_fetch_kib=fk, copy_write_kib=wk,
                fetch_scale=round(ff, 6), write_scale=round(wf, 6),
                hbm_bytes_per_launch=round(avg) if avg is not None else None, kernels=kernels)


def traffic_md(rec, commands):
    lines = ["Commands (from the repository root, on one MI355X):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", f"Calibration: a {rec['copy_bytes']} byte device copy reads FETCH_SIZE = {rec['copy_fetch_kib']:.1f} KiB "
              f"and WRITE_SIZE = {rec['copy_write_kib']:.1f} KiB, so FETCH_SIZE is scaled by {rec['fetch_scale']} and "
              f"WRITE_SIZE by {rec['write_scale']} (bytes = KiB x 1024 x scale).", "",
              f"Workload `{rec['workload']}`; linear-layer source hash `{rec['kernel_source_sha']}`.", "",
              "| kernel | grid (threads) | launches | HBM read MB | HBM write MB | total MB |",
              "|---|---:|---:|---:|---:|---:|"]
    for k in rec["kernels"]:
        lines.append(f"| `{k['kernel']}` | {k['grid']} | {k['launches']} | {k['fetch_bytes'] / 1e6:.1f} | "
                     f"{k['write_bytes'] / 1e6:.1f} | {k['hbm_bytes'] / 1e6:.1f} |")
    lines += ["", f"Average over the `{rec['kernel']}` launches of one step: "
              f"{rec['hbm_bytes_per_launch'] / 1e6:.1f} MB per launch."]
    return "\n".join(lines) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--commands", nargs="+", required=True)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", default="k_linear")
    t.add_argument("--json-out", default="")
    t.add_argument("--md-out", default="")
    t.add_argument("--commands", nargs="*", default=[])
    a = p.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats(a.dir, a.commands))
    else:
        rec = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.workload, a.kernel)
        text = json.dumps(rec, indent=1)
        if a.json_out:
            with open(a.json_out, "w") as fh:
                fh.write(text + "\n")
        if a.md_out:
            with open(a.md_out, "w") as fh:
                fh.write(traffic_md(rec, a.commands))
        print(text)


if __name__ == "__main__":
    main()
