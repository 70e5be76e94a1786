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


def library_source_sha():
    """Hash of every source of the library; the per-kernel counter summary records it,
    so figures taken on other kernels are not reused."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "integer_rank_adaptation_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".inc")):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
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
    ff, fk = copy_factor(cf_dir, "FETCH_SIZE", copy_bytes) if cf_dir else (None, None)
    wf, wk = copy_factor(cw_dir, "WRITE_SIZE", copy_bytes) if cw_dir else (None, None)
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


# The kernels of one step of the benchmark, in launch order per layer (the merge's three
# kernels, then the linear layer).  Their launches cycle through the layers in order, so
# launch k of a kernel belongs to layer k mod L.
STEP_KERNELS = ("k_adapt_mfma", "k_adapt_generic", "k_row_range", "k_mul_params", "k_quant_mul", "k_quant_shift",
                "k_linear", "k_linear_planes", "k_linear_skinny", "k_linear_skinny_planes")
CLOCK_HZ = 2.4e9
SIMDS = 256 * 4
XCDS = 8


def _by_layer(rows, layers, value):
    """{kernel base name: [per-layer list of values]} for the step kernels, launch k of a
    kernel -> layer k mod len(layers); other kernels (set-up) are left out."""
    seq = collections.OrderedDict()
    for r in sorted(rows, key=lambda r: r["dispatch"]):
        base = r["name"].split("<")[0]
        if base not in STEP_KERNELS:
            continue
        seq.setdefault(r["name"], []).append(value(r))
    out = {}
    for name, vals in seq.items():
        per = [[] for _ in layers]
        for k, v in enumerate(vals):
            per[k % len(layers)].append(v)
        out[name] = per
    return out


def read_trace_rows(d):
    rows = list(csv.DictReader(open(_one(d, "*kernel_trace.csv"))))
    return [dict(name=short_name(r["Kernel_Name"]), us=(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3,
                 dispatch=int(r["Dispatch_Id"])) for r in rows]


def read_counter_rows(d):
    rows = list(csv.DictReader(open(_one(d, "*counter_collection.csv"))))
    return [dict(name=short_name(r["Kernel_Name"]), counter=r["Counter_Name"], v=float(r["Counter_Value"]),
                 dispatch=int(r["Dispatch_Id"])) for r in rows]


def counters(trace_dir, pmc_dirs, cf_dir, cw_dir, copy_bytes, workload, layers, commands):
    """Per layer and kernel of the step: median duration (kernel trace), HBM bytes
    (FETCH_SIZE / WRITE_SIZE scaled by a plain copy of known size), and the SQ / GRBM
    counters of the other runs; derived: counter GB/s, the clock during the kernel
    (GRBM_GUI_ACTIVE / duration), the vector-ALU issue fraction (4 cycles per wave64
    VALU instruction on a 16-lane SIMD; of the cycles at the measured clock, and of the
    2.4 GHz peak) and the matrix-core busy fraction."""
    import statistics

    ff, fk = copy_factor(cf_dir, "FETCH_SIZE", copy_bytes) if cf_dir else (None, None)
    wf, wk = copy_factor(cw_dir, "WRITE_SIZE", copy_bytes) if cw_dir else (None, None)
    dur = _by_layer(read_trace_rows(trace_dir), layers, lambda r: r["us"])
    vals = collections.defaultdict(dict)  # kernel -> counter -> per-layer lists
    for d in pmc_dirs:
        rows = read_counter_rows(d)
        for cname in sorted({r["counter"] for r in rows}):
            sel = [r for r in rows if r["counter"] == cname]
            for kname, per in _by_layer(sel, layers, lambda r: r["v"]).items():
                vals[kname][cname] = per
    med = lambda xs: statistics.median(xs) if xs else None
    per_layer = {L: {} for L in layers}
    for kname, per in dur.items():
        for li, L in enumerate(layers):
            rec = dict(us=round(med(per[li]), 3) if per[li] else None, launches=len(per[li]))
            cv = {c: med(v[li]) for c, v in vals.get(kname, {}).items() if v[li]}
            if "FETCH_SIZE" in cv and ff:
                rec["fetch_bytes"] = round(cv["FETCH_SIZE"] * 1024 * ff)
            if "WRITE_SIZE" in cv and wf:
                rec["write_bytes"] = round(cv["WRITE_SIZE"] * 1024 * wf)
            if rec["us"] and "fetch_bytes" in rec and "write_bytes" in rec:
                rec["hbm_bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
                rec["counter_GBps"] = round(rec["hbm_bytes"] / (rec["us"] * 1e-6) / 1e9, 1)
                rec["counter_pct_hbm_peak"] = round(100 * rec["counter_GBps"] / 8000.0, 2)
            for c, v in cv.items():
                if c not in ("FETCH_SIZE", "WRITE_SIZE"):
                    rec[c] = v
            # GRBM_GUI_ACTIVE comes summed over the XCDs: cycles of the kernel = value / XCDS.
            # It also counts a few microseconds of dispatch around each launch (short kernels
            # read above 2.4 GHz), so the clock is derived only for launches of 100 us or
            # more, and is an upper bound there.
            cycles = cv["GRBM_GUI_ACTIVE"] / XCDS if cv.get("GRBM_GUI_ACTIVE") else None
            if rec["us"] and cycles and rec["us"] >= 100:
                rec["clock_GHz"] = round(cycles / (rec["us"] * 1e-6) / 1e9, 3)
            if rec["us"] and cv.get("SQ_INSTS_VALU"):
                rec["valu_frac_of_peak"] = round(cv["SQ_INSTS_VALU"] * 4 / (rec["us"] * 1e-6 * CLOCK_HZ * SIMDS), 4)
                if cycles:
                    rec["valu_frac_at_clock"] = round(cv["SQ_INSTS_VALU"] * 4 / (cycles * SIMDS), 4)
            if cv.get("SQ_VALU_MFMA_BUSY_CYCLES") and cycles:
                rec["mfma_busy_frac"] = round(cv["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * SIMDS), 4)
            per_layer[L][kname] = rec
    out = dict(workload=workload, library_source_sha=library_source_sha(), command=commands,
               calibration=dict(copy_bytes=copy_bytes, copy_fetch_kib=fk, copy_write_kib=wk,
                                fetch_scale=round(ff, 6) if ff else None, write_scale=round(wf, 6) if wf else None),
               per_layer=per_layer)
    # rooflines of the merge's quantize kernel (HBM) and adaptation kernel (vector ALU),
    # aggregated over the step's layers
    for key, prefix, unit in (("roofline_merge", ("k_quant_mul", "k_quant_shift"), "GB/s"),
                              ("roofline_adapt", ("k_adapt_mfma", "k_adapt_generic"), "valu")):
        keyed = [(k, r) for L in layers for k, r in per_layer[L].items() if k.startswith(prefix) and r.get("us")]
        if not keyed:
            continue
        recs = [r for _, r in keyed]
        kname = ", ".join(sorted({k for k, _ in keyed}))
        t = sum(r["us"] for r in recs) * 1e-6
        if unit == "GB/s" and all("hbm_bytes" in r for r in recs):
            b = sum(r["hbm_bytes"] for r in recs)
            out[key] = dict(bound="hbm", kernel=kname, achieved=round(b / t / 1e9, 1), peak=8000.0,
                            unit="GB/s", frac=round(b / t / 1e9 / 8000.0, 4), traffic=round(b / len(layers)),
                            source="rocprofv3 FETCH_SIZE + WRITE_SIZE (copy-calibrated) over kernel-trace time, "
                                   "summed over the step's layers")
        elif unit == "valu" and all("SQ_INSTS_VALU" in r for r in recs):
            n = sum(r["SQ_INSTS_VALU"] for r in recs)
            lane = n * 64 / t / 1e12
            out[key] = dict(bound="alu", kernel=kname, achieved=round(lane, 2), peak=39.32,
                            unit="T lane-instructions/s (vector ALU)", frac=round(lane / 39.32, 4), traffic=None,
                            source="rocprofv3 SQ_INSTS_VALU (wave64 instructions) x 64 lanes over kernel-trace "
                                   "time; peak 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz")
    return out


def counters_md(rec):
    """Markdown summary of a per-kernel counter record (the output of `counters`)."""
    cal = rec["calibration"]
    lines = ["Commands (from the repository root, on one MI355X):", ""]
    lines += ["    " + c for c in rec.get("command", [])]
    lines += ["", f"Workload `{rec['workload']}`; library source hash `{rec['library_source_sha']}`.",
              (f"HBM bytes = FETCH_SIZE x {cal['fetch_scale']} + WRITE_SIZE x {cal['write_scale']} (KiB x 1024), "
               f"calibrated on a {cal['copy_bytes']} byte device copy." if cal.get("fetch_scale") else
               "Kernel trace only (no counter passes)."),
              "GRBM_GUI_ACTIVE is summed over the 8 XCDs and includes a few us of dispatch per launch (clock = value / 8 / duration, an upper bound, given for launches of 100 us or more); VALU fraction of peak = "
              "SQ_INSTS_VALU x 64 lanes / duration / 39.32 T lane-instructions/s; MfmaUtil and VALUBusy are "
              "rocprofv3's derived percentages.", "",
              "| layer | kernel | us (trace) | HBM MB | counter GB/s | % of 8 TB/s | VALU insts / elem | "
              "VALU % of peak | VALUBusy % | MfmaUtil % | clock GHz |",
              "|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for L, ks in rec["per_layer"].items():
        for k, r in ks.items():
            hb = r.get("hbm_bytes")
            clk = r.get("clock_GHz")
            epe = r.get("valu_per_elem")
            lines.append("| %s | `%s` | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
                L, k, f"{r['us']:.1f}" if r.get("us") else "-", f"{hb / 1e6:.1f}" if hb else "-",
                f"{r['counter_GBps']:.0f}" if r.get("counter_GBps") else "-",
                f"{r['counter_pct_hbm_peak']:.1f}" if r.get("counter_pct_hbm_peak") else "-",
                f"{epe:.1f}" if epe else "-",
                f"{100 * r['valu_frac_of_peak']:.1f}" if r.get("valu_frac_of_peak") else "-",
                f"{r['VALUBusy']:.1f}" if r.get("VALUBusy") is not None else "-",
                f"{r['MfmaUtil']:.1f}" if r.get("MfmaUtil") is not None else "-",
                f"{clk:.2f}" if clk else "-"))
    for key in ("roofline_merge", "roofline_adapt"):
        if key in rec:
            r = rec[key]
            lines += ["", f"`{key}`: {r['kernel']} -- {r['achieved']} {r['unit']} of {r['peak']} "
                      f"(frac {r['frac']}); {r['source']}."]
    return "\n".join(lines) + "\n"


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
    c = sub.add_parser("counters")
    c.add_argument("--trace", required=True)
    c.add_argument("--pmc", nargs="*", default=[])
    c.add_argument("--copy-fetch", default="")
    c.add_argument("--copy-write", default="")
    c.add_argument("--copy-bytes", type=int, default=0)
    c.add_argument("--workload", required=True)
    c.add_argument("--layers", required=True, help="comma-separated layer names in step order")
    c.add_argument("--elems", default="", help="comma-separated weights per layer (VALU instructions per weight)")
    c.add_argument("--json-out", default="")
    c.add_argument("--md-out", default="")
    c.add_argument("--commands", nargs="*", default=[])
    a = p.parse_args(argv)
    if a.cmd == "counters":
        layers = a.layers.split(",")
        rec = counters(a.trace, a.pmc, a.copy_fetch, a.copy_write, a.copy_bytes, a.workload, layers, a.commands)
        if a.elems:
            for L, e in zip(layers, [float(x) for x in a.elems.split(",")]):
                for r in rec["per_layer"][L].values():
                    if r.get("SQ_INSTS_VALU"):
                        r["valu_per_elem"] = round(r["SQ_INSTS_VALU"] * 64 / e, 2)
        text = json.dumps(rec, indent=1)
        if a.json_out:
            with open(a.json_out, "w") as fh:
                fh.write(text + "\n")
        if a.md_out:
            with open(a.md_out, "w") as fh:
                fh.write(counters_md(rec))
        print(text)
        return
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
