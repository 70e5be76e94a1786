"""Benchmark of the IntLoRA hot path on one MI355X.

One step = the whole path over one batch of the workload: for every layer, the
MUL (or SHIFT) merge of the trained LoRA factors into the quantized base (R*
regeneration, adaptation term, row statistics, quantize + integer Hadamard / shift)
followed by the integer linear layer that consumes the merged integers (int8 MFMA,
dequantized bf16 output).  Inputs (quantized base, LoRA factors, quantized
activations) are resident in HBM before the timed region.

Default workload: the FLUX-like DiT block linears (hidden 3072; qkv 9216x3072,
out 3072x3072, mlp 12288x3072 and 3072x12288), W4A8, MUL with a 4-bit adaptation
term, rank 32, 4608 tokens.

Printed (rank 0, one JSON line): value = 100 * T_roof / T_step, where T_roof is the
step's time at MI355X peak (merge algorithmic bytes at 8 TB/s HBM plus, per linear
layer, the longer of its products -- each merged integer times each activation counted
once as an int8 multiply-add -- at 5.0 POP/s and its bytes at 8 TB/s) and T_step the
measured time of one step.  T_roof is a
constant of the workload, so value is inversely proportional to the step time.
T_step is that of the fastest of the measured schedules of the same kernels whose
outputs equal the sequential step's (sequential; pipelined, the merges on a second
stream; each also replayed from a HIP graph), named in `schedule`; every schedule's
time is listed, and the roofline of the dominant kernel comes from the per-launch
events of the sequential step.  Per-layer merge GB/s and GEMM TOP/s are listed
alongside.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "merge GB/s + W8A8/W4A8 GEMM int8 TOPS (% of MI355X peak) per layer shape"
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0
FP32_MFMA_TFLOPS = 157.3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=3)
    p.add_argument("--tokens", type=int, default=0, help="override M (0: the workload's first)")
    p.add_argument("--cpu-sample", type=float, default=0.0,
                   help="fraction of rows/tokens the oracle processes (0: auto, about 15 s)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--json-out", default="")
    p.add_argument("--no-overlap", action="store_true",
                   help="skip the pipelined step (merges on a second stream, each layer's linear layer "
                        "waiting only for its own merge), which is timed beside the sequential one")
    p.add_argument("--no-ptq", action="store_true",
                   help="skip the QLoRA-style comparison (MUL workloads): the dequantize / add / requant "
                        "path timed on the same layers, and both paths' weight error")
    p.add_argument("--no-fused", action="store_true",
                   help="skip the fused single-pass MUL merge (U kept on chip, no workspace), timed on the same "
                        "layers against the three-kernel merge")
    p.add_argument("--no-codes", action="store_true",
                   help="skip the merge-on-load path (MUL, 4-bit U and base codes): the merge keeping U's "
                        "codes and the linear layer forming m from them, timed on the same layers")
    p.add_argument("--no-ste", action="store_true",
                   help="skip the straight-through backward (a synthetic dL/dW' per layer, dA and dB)")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the step captured in a HIP graph and replayed (reported beside the eager step)")
    p.add_argument("--no-aux-laws", action="store_true",
                   help="skip the merge timed under the other auxiliary laws (Gaussian, Cauchy, Student-t(2))")
    p.add_argument("--int16-layout", action="store_true",
                   help="MUL: keep the merged integers as int16 (converted to byte planes inside the linear "
                        "layer) instead of the byte-plane storage")
    p.add_argument("--kernel-runs", type=int, default=100,
                   help="runs per kernel for the per-kernel medians (merge warm, merge cold, linear layer)")
    p.add_argument("--flush-mib", type=int, default=1024,
                   help="bytes streamed through HBM before each cold merge run (defeats the 256 MB Infinity Cache)")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the merge-only sweep over the 32 transformer blocks x 7 matrices of the "
                        "Llama-3-8B-shaped workload")
    p.add_argument("--sweep-blocks", type=int, default=32, help="transformer blocks in the merge-only sweep")
    p.add_argument("--no-grouped", action="store_true",
                   help="Llama-3-8B-shaped block: skip the step with q/k/v and gate/up each run as one linear-layer "
                        "call over their concatenated rows")
    p.add_argument("--no-library-gemm", action="store_true",
                   help="skip the context timing of the vendor library's int8 GEMM (torch._int_mm) on the same "
                        "int8 operands")
    p.add_argument("--mode-index", type=int, default=0,
                   help="which of the workload's merge modes to time (the SD-v1.5 640-channel set has MUL "
                        "then SHIFT)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (counter calibration) and exit")
    return p.parse_args()


def copy_probe(mib):
    """A plain copy kernel of known size: the HBM counters of this run calibrate the
    FETCH_SIZE / WRITE_SIZE readings of the library's kernels."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n}))


def merge_alg_bytes(d, n, r, w_bits, mode):
    """Bytes the merge itself must move: W_round in, merged integers out, A and B,
    and the per-row vectors (z, s, c in; s_bar, z_bar out).  R is regenerated."""
    code_in = d * n * (0.5 if w_bits == 4 else 1.0)
    if mode == "mul":
        out = d * n * 2.0
    else:
        out = d * n * (0.5 if w_bits == 4 else 1.0)
    return code_in + out + 4.0 * d * r + 4.0 * r * n + 20.0 * d


def gemm_exec_ops(M, d, n, mode, planes=None):
    """int8 MFMA operations the linear layer executes: one pass per byte plane it
    multiplies (MUL: two, or one when the byte-plane storage has every high plane zero)."""
    passes = (2 if mode == "mul" else 1) if planes is None else planes
    return 2.0 * M * d * n * passes


def gemm_alg_bytes(M, d, n, mode, w_bits, nplanes):
    """HBM bytes the linear layer needs: the int8 activations, the stored weights (MUL:
    one byte per multiplied plane, or the int16 integers; SHIFT: the w_bits codes) and
    the bf16 outputs."""
    if mode == "mul":
        wb = 2.0 if nplanes is None else float(nplanes)
    else:
        wb = w_bits / 8.0
    return float(M) * n + d * n * wb + 2.0 * M * d


def planes_multiplied(M, d, n, any_code, torch):
    """Byte planes the linear layer multiplies on the byte-plane storage: one when every
    plane code is 0 and (above 32 tokens) its 256-output tiles take fewer rounds of the
    persistent grid than the two-plane tiles -- the library's launch rule -- else two.
    (At most 32 tokens the kernel decides per block of 16 rows; the workloads' codes are
    uniform over a layer, so the layer-wide answer is the same.)"""
    if any_code:
        return 2
    if M <= 32:
        return 1
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tm = -(-M // 256)
    t2, tn, kt = tm * -(-d // 128), tm * -(-d // 256), -(-n // 64)
    g = cus if kt >= 3 and t2 > cus else t2
    return 1 if -(-tn // g) < -(-t2 // g) else 2


def merged_m(lay, torch):
    """The merged integers of a layer's MUL output as int32 (from either storage)."""
    o = lay["out"]
    if "planes" not in o:
        return o["m"].to(torch.int32)
    n = o["planes"].shape[1] // 2
    g = o["planes"].view(torch.int8).to(torch.int32)
    hi, lo = g[:, :n], g[:, n:]  # per row: the high plane, then the low plane
    return 256 * hi + lo + 128 * ((o["code"].to(torch.int32) >> 1) & 1)[:, None]


def traffic_from_profile(workload_name, kernel_prefix):
    """HBM bytes per launch of the dominant kernel (mean over the step's layers) from the
    committed counter summary, if it was taken on the current library source; else None."""
    path = os.path.join(ROOT, "profiles", workload_name + "_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    from integer_rank_adaptation_amd.profiling import library_source_sha

    if rec.get("library_source_sha") != library_source_sha() or rec.get("workload") != workload_name:
        return None
    vals = [r["hbm_bytes"] for ks in rec["per_layer"].values() for k, r in ks.items()
            if k.startswith(kernel_prefix) and r.get("hbm_bytes")]
    return round(sum(vals) / len(vals)) if vals else None


def ptq_comparison(args, wl, layers, ws, ops, B, synth, torch, dev, stream, rows_per_layer=64):
    """The flow IntLoRA removes, on the same layers: dequantize, add R* + AB in binary32,
    requantize each row at the base's bit width (intlora_merge_ptq).  Times it like the
    merge (whole layers, events on the same stream) and compares both paths' merged
    weights with the binary64 adapted weight s w + R* + AB on sampled rows."""
    outs = [None] * len(layers)

    def run():
        for k, lay in enumerate(layers):
            outs[k] = ops.merge_ptq(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, wl.w_bits, synth.PHILOX_SEED,
                                    lay["lid"], ws=ws, out=outs[k])

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ptq_ms = e0.elapsed_time(e1) / args.steps

    def unpack(codes, n):
        if codes.shape[1] == n:
            return codes.to(torch.int64)
        c = codes.to(torch.int64)
        return torch.stack([c & 15, c >> 4], dim=2).reshape(codes.shape[0], n)

    per = []
    for k, lay in enumerate(layers):
        L = lay["L"]
        rows = torch.linspace(0, L.d - 1, rows_per_layer, device=dev).round().to(torch.int64).unique()
        c = lay["st"]["c"]
        R = torch.empty((L.d, L.n), dtype=torch.float32, device=dev)
        B.intlora_gen_r(B.desc(L.d, L.n, wl.r, wl.w_bits, synth.PHILOX_SEED, lay["lid"]), c, R)
        w = unpack(lay["st"]["wround"][rows], L.n) - lay["st"]["z"][rows].to(torch.int64)[:, None]
        target = (lay["st"]["s"][rows].double()[:, None] * w.double() + R[rows].double()
                  + lay["Ag"][rows].double() @ lay["Bg"].double())
        m = merged_m(lay, torch)[rows].double()
        intlora = lay["out"]["sbar"][rows].double()[:, None] * m
        code = unpack(outs[k]["code"][rows], L.n)
        ptqw = outs[k]["s"][rows].double()[:, None] * (code - outs[k]["z"][rows].to(torch.int64)[:, None]).double()
        tn = torch.linalg.norm(target)
        per.append(dict(layer=L.name, rel_err_intlora=float(torch.linalg.norm(intlora - target) / tn),
                        rel_err_ptq=float(torch.linalg.norm(ptqw - target) / tn), rows=int(rows.numel())))
        del R
    code_b = 0.5 if wl.w_bits == 4 else 1.0
    alg = sum(lay["L"].d * lay["L"].n * 2 * code_b for lay in layers)  # base codes in, new codes out
    return dict(kind="dequantize + add R* + AB (binary32) + per-row RTN requant at %d bits" % wl.w_bits,
                error_note="errors against s w + R* + AB with the synthetic adapter, whose B has variance 1e-3 "
                           "(the workload's N(0, 1e-3) read as a variance): AB is then several times larger than "
                           "W, which widens U's range and the MUL step s_bar; they say little about the method, "
                           "whose training starts from B = 0",
                ptq_merge_us_per_step=round(ptq_ms * 1e3, 1),
                alg_GBps=round(alg / (ptq_ms * 1e-3) / 1e9, 1),
                pct_hbm_peak=round(100 * alg / (ptq_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                bound="alu (the adaptation kernel's Philox, ln and rank-r work)", per_layer=per)


AUX_LAW_NAMES = {1: "gaussian", 2: "cauchy", 3: "student_t2"}


def aux_laws_measure(args, wl, layers, ops, synth, torch, dev, ws, stream, mode, mbits):
    """The step's merge under each other auxiliary law of the distribution ablation: the
    same layers set up again with that law (untimed), then the MUL or SHIFT merge timed
    like the main step's (whole layers, events on the same stream)."""
    res = {}
    for dist, name in AUX_LAW_NAMES.items():
        sts, outs = [], []
        for lay in layers:
            Wg = torch.from_numpy(lay["W"]).to(dev)
            sts.append(ops.setup_layer(Wg, wl.w_bits, synth.PHILOX_SEED, lay["lid"], synth.ALPHA, aux_dist=dist))
            del Wg
            outs.append(None)

        def run():
            for k, lay in enumerate(layers):
                if mode == "mul":
                    outs[k] = ops.merge_mul(sts[k], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED,
                                            lay["lid"], ws=ws, out=outs[k])
                else:
                    outs[k] = ops.merge_shift(sts[k], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED,
                                              lay["lid"], ws=ws, out=outs[k])

        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        alg = sum(merge_alg_bytes(lay["L"].d, lay["L"].n, wl.r, wl.w_bits, mode) for lay in layers)
        res[name] = {"merge_us_per_step": round(ms * 1e3, 1), "alg_GBps": round(alg / (ms * 1e-3) / 1e9, 1)}
        del sts, outs
    res["bound"] = "alu (the sampler's ln, sqrt, cos / sin / tan in binary64 replace the Laplace ln)"
    return res


def fused_measure(args, wl, layers, ops, synth, torch, dev, stream, mbits):
    """Fused single-pass MUL merge on the same layers (no workspace: U stays on chip),
    timed like the main step's merges; its merged integers are checked equal to the main
    path's, layer by layer."""
    outs = [None] * len(layers)

    def run(events=None):
        for k, lay in enumerate(layers):
            if events is not None:
                events[k][0].record(stream)
            outs[k] = ops.merge_mul_fused(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED,
                                          lay["lid"], out=outs[k])
            if events is not None:
                events[k][1].record(stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in layers] for _ in range(args.steps)]
    for s_ in range(args.steps):
        run(ev[s_])
    torch.cuda.synchronize()
    per = []
    tot = 0.0
    for k, lay in enumerate(layers):
        us = sum(ev[s_][k][0].elapsed_time(ev[s_][k][1]) for s_ in range(args.steps)) / args.steps * 1e3
        tot += us
        per.append(dict(layer=lay["L"].name, fused_merge_us=round(us, 2),
                        same_m_as_three_kernel_merge=bool(torch.equal(outs[k]["m"].to(torch.int32),
                                                                      merged_m(lay, torch)))))
    code_b = 0.5 if wl.w_bits == 4 else 1.0
    alg = sum(lay["L"].d * lay["L"].n * (code_b + 2.0) for lay in layers)  # base codes in, int16 m out
    return dict(us_per_step=round(tot, 1), alg_GBps=round(alg / (tot * 1e-6) / 1e9, 1),
                pct_hbm_peak=round(100 * alg / (tot * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                bound="L2 and alu (B re-read per row block; rank-r chain on the vector ALU)", per_layer=per)


def codes_measure(args, wl, layers, ops, synth, torch, dev, ws, stream, mbits):
    """Merge-on-load path on the same layers and tokens: the MUL merge storing U's 4-bit
    codes (no int16 m) and the linear layer forming m = (U_round - z_bar)(W_round - z)
    per tile.  Timed like the main step; its outputs are checked equal to the main
    path's (same Y bits), layer by layer."""
    outs = []
    for lay in layers:
        L = lay["L"]
        outs.append(dict(ucode=torch.empty((L.d, L.n // 2), dtype=torch.uint8, device=dev),
                         sbar=torch.empty(L.d, dtype=torch.float32, device=dev),
                         zbar=torch.empty(L.d, dtype=torch.int32, device=dev)))
    Ys = [torch.empty_like(lay["Y"]) for lay in layers]

    def step(events=None):
        for k, lay in enumerate(layers):
            if events is not None:
                events[k][0].record(stream)
            ops.merge_mul_codes(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"],
                                ws=ws, out=outs[k])
            if events is not None:
                events[k][1].record(stream)
            ops.linear_codes(lay["xq"], lay["sx"], outs[k]["ucode"], lay["st"]["wround"], lay["st"]["z"],
                             outs[k]["zbar"], outs[k]["sbar"], lay["L"].d, out=Ys[k])
            if events is not None:
                events[k][2].record(stream)

    def merge_fn(k):
        lay = layers[k]
        if mode == "mul":
            ops.merge_mul(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"], ws=ws,
                          out=lay["out"])
        else:
            ops.merge_shift(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"], ws=ws,
                            out=lay["out"])

    def gemm_fn(k):
        lay = layers[k]
        ops.linear(lay["xq"], lay["sx"], lay["rs"], lay["wfmt"], lay["out"]["m"], lay["out"]["sbar"], lay["L"].d,
                   out=lay["Y"], split=lay["out"].get("split"))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers] for _ in range(args.steps)]
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s_ in range(args.steps):
        step(ev[s_])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per = []
    for k, lay in enumerate(layers):
        mm = sum(ev[s_][k][0].elapsed_time(ev[s_][k][1]) for s_ in range(args.steps)) / args.steps
        gm = sum(ev[s_][k][1].elapsed_time(ev[s_][k][2]) for s_ in range(args.steps)) / args.steps
        same = bool(torch.equal(Ys[k], lay["Y"]))
        per.append(dict(layer=lay["L"].name, merge_codes_us=round(mm * 1e3, 2), gemm_codes_us=round(gm * 1e3, 2),
                        same_Y_as_int16_path=same))
    merge_us = sum(p["merge_codes_us"] for p in per)
    gemm_us = sum(p["gemm_codes_us"] for p in per)
    alg = sum(lay["L"].d * lay["L"].n * 1.0 for lay in layers)  # 4-bit base codes in, 4-bit U codes out
    ops_exec = sum(2.0 * 2 * lay["xq"].shape[0] * lay["L"].d * lay["L"].n for lay in layers)  # two int8 planes
    return dict(ms_per_step=round(ms, 4), merge_codes_us_per_step=round(merge_us, 1),
                merge_codes_alg_GBps=round(alg / (merge_us * 1e-6) / 1e9, 1),
                gemm_codes_us_per_step=round(gemm_us, 1),
                gemm_codes_exec_TOPS=round(ops_exec / (gemm_us * 1e-6) / 1e12, 1),
                gemm_codes_pct_int8_peak=round(100 * ops_exec / (gemm_us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 2),
                per_layer=per, weight_bytes_per_adapter="0.5 B/weight (U codes) vs 2 B/weight (int16 m)")


def ste_measure(args, wl, layers, ops, torch, dev, stream):
    """The straight-through backward of every layer (dA = D B^T, dB = A^T D with
    D = G.[w != 0]) on a seeded synthetic gradient G ~ N(0, 1e-6) per layer, timed like
    the merge.  Two bounds per element: one pass over G (4 B) and its code (HBM), and
    the two products' 4 r flops on the fp32 matrix cores (157.3 TFLOP/s); the fused
    kernel reads G and the codes once."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    Gs = [torch.randn((lay["L"].d, lay["L"].n), generator=gen, device=dev, dtype=torch.float32) * 1e-3
          for lay in layers]
    outs = [None] * len(layers)

    def run():
        for k, lay in enumerate(layers):
            outs[k] = ops.ste_backward(lay["st"], lay["Ag"], lay["Bg"], Gs[k], wl.w_bits, out=outs[k])

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    code_b = 0.5 if wl.w_bits == 4 else 1.0
    one_pass = sum(lay["L"].d * lay["L"].n * (4 + code_b) for lay in layers)
    flops = sum(4.0 * lay["L"].d * lay["L"].n * wl.r for lay in layers)
    del Gs
    t_hbm = one_pass / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (FP32_MFMA_TFLOPS * 1e12)
    return dict(us_per_step=round(ms * 1e3, 1), one_pass_GBps=round(one_pass / (ms * 1e-3) / 1e9, 1),
                one_pass_pct_hbm=round(100 * one_pass / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                fp32_mfma_TFLOPs=round(flops / (ms * 1e-3) / 1e12, 1),
                bound="mfma" if t_mfma >= t_hbm else "hbm",
                frac_of_bound=round(max(t_hbm, t_mfma) / (ms * 1e-3), 3))


def kernel_medians(args, layers, merge_fn, gemm_fn, torch, dev, stream):
    """Per-layer kernel times, median of `args.kernel_runs` runs each (after 10 untimed
    ones): the merge warm (back to back, so a layer's inputs may sit in the 256 MB
    Infinity Cache), the merge cold (a 1 GiB buffer is written through HBM before each
    run, evicting L2 and the Infinity Cache), and the linear layer (warm: it is bound by
    the matrix cores).  HIP events on the stream the kernels run on."""
    runs = max(1, args.kernel_runs)
    flush = torch.empty(max(1, args.flush_mib) << 20, dtype=torch.uint8, device=dev)

    def timed(fn, k, cold):
        for _ in range(10):
            fn(k)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        for e0, e1 in ev:
            if cold:
                flush.fill_(1)
            e0.record(stream)
            fn(k)
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

    out = []
    for k in range(len(layers)):
        out.append(dict(merge_warm_us=round(timed(merge_fn, k, False), 2),
                        merge_cold_us=round(timed(merge_fn, k, True), 2),
                        gemm_us=round(timed(gemm_fn, k, False), 2)))
    del flush
    return out


def int16_layout_medians(args, layers, ops, synth, wl, mbits, ws, torch, dev, stream):
    """The linear layer on the same merged integers stored as int16 (the layer converts
    them to byte planes after its LDS reads): median of `args.kernel_runs` runs per layer,
    the outputs checked equal to the byte-plane path's."""
    out = []
    for lay in layers:
        L = lay["L"]
        g = ops.merge_mul(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"], ws=ws)
        Y = torch.empty_like(lay["Y"])

        def fn():
            ops.linear(lay["xq"], lay["sx"], lay["rs"], 16, g["m"], g["sbar"], L.d, out=Y, split=g["split"])

        for _ in range(10):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(max(1, args.kernel_runs))]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        assert torch.equal(Y, lay["Y"]), "int16 layout and byte planes disagree"
        out.append(round(float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3, 2))
        del g, Y
    return out


def library_gemm_medians(args, layers, mode, w_bits, planes, torch, stream):
    """For context: the vendor library's int8 GEMM (torch._int_mm: int32 accumulators, no
    epilogue, no bf16 output) on the same activations and merged integers, where those
    are int8 (MUL with every high byte zero, or SHIFT at 8 bits).  Median of
    `args.kernel_runs` runs per layer; None for layers it cannot take."""
    out = []
    for lay in layers:
        L = lay["L"]
        o = lay["out"]
        w8 = None
        if mode == "mul" and planes and not bool(o["code"].any()):
            w8 = o["planes"].view(L.d, 2, L.n)[:, 1, :].contiguous().view(torch.int8)  # the low planes
        elif mode == "shift" and w_bits == 8:
            w8 = o["m"].view(torch.int8).view(L.d, L.n)
        if w8 is None or lay["xq"].shape[0] <= 16:
            out.append(None)
            continue
        wt = w8.t()

        def fn():
            return torch._int_mm(lay["xq"], wt)

        try:
            for _ in range(10):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(max(1, args.kernel_runs))]
            for e0, e1 in ev:  # torch's current stream, as every other timing here
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            out.append(round(float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3, 2))
        except RuntimeError:
            out.append(None)
    return out


def profile_counters(workload_name):
    """Per-kernel counter figures from the committed rocprofv3 summary of this workload
    (profiles/<workload>_counters.json), if it was taken on the current kernel sources;
    else None."""
    path = os.path.join(ROOT, "profiles", workload_name + "_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    from integer_rank_adaptation_amd.profiling import library_source_sha

    if rec.get("library_source_sha") != library_source_sha() or rec.get("workload") != workload_name:
        return None
    return rec


# Llama-3-8B-shaped block: the projections that read the same activations
SHARED_INPUT_GROUPS = {4: (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))}


def grouped_measure(args, wl, layers, ops, synth, torch, dev, stream, mbits, ws):
    """The projections of a block that read the same activations (q, k, v; gate, up) as
    one linear-layer call each: every matrix is merged on its own (MUL, byte planes) into
    its row slice of the group's buffers, and the group's linear layer runs once over the
    concatenated rows with the first member's activations.  Timed like the step (events
    around every merge and every group call); each group's outputs are checked equal to
    the per-matrix calls on the same activations."""
    by_name = {lay["L"].name: lay for lay in layers}
    groups = []
    for names in SHARED_INPUT_GROUPS[wl.index]:
        mem = [by_name[nm] for nm in names]
        n = mem[0]["L"].n
        D = sum(l["L"].d for l in mem)
        buf = dict(planes=torch.empty((D, 2 * n), dtype=torch.uint8, device=dev),
                   sbar=torch.empty(D, dtype=torch.float32, device=dev),
                   zbar=torch.empty(D, dtype=torch.int32, device=dev),
                   code=torch.empty(D, dtype=torch.uint8, device=dev))
        outs, r0 = [], 0
        for l in mem:
            d = l["L"].d
            outs.append(dict(planes=buf["planes"][r0:r0 + d], sbar=buf["sbar"][r0:r0 + d],
                             zbar=buf["zbar"][r0:r0 + d], code=buf["code"][r0:r0 + d],
                             sat=torch.zeros(2, dtype=torch.int64, device=dev)))
            r0 += d
        Y = torch.empty((mem[0]["xq"].shape[0], D), dtype=torch.int16, device=dev)
        groups.append(dict(mem=mem, buf=buf, outs=outs, D=D, Y=Y, lay0=mem[0]))

    def run(events=None):
        for gi, g in enumerate(groups):
            if events is not None:
                events[gi][0].record(stream)
            for l, o in zip(g["mem"], g["outs"]):
                ops.merge_mul_planes(l["st"], l["Ag"], l["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, l["lid"],
                                     ws=ws, out=o)
            if events is not None:
                events[gi][1].record(stream)
            x = g["lay0"]
            ops.linear(x["xq"], x["sx"], x["rs"], ops.B.INTLORA_W_INT16_PLANES, g["buf"]["planes"], g["buf"]["sbar"],
                       g["D"], out=g["Y"], split=g["buf"]["code"])
            if events is not None:
                events[gi][2].record(stream)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    same = True
    for g in groups:  # per-matrix calls on the group's activations give the same outputs
        x = g["lay0"]
        r0 = 0
        for l, o in zip(g["mem"], g["outs"]):
            d = l["L"].d
            Yk = torch.empty((x["xq"].shape[0], d), dtype=torch.int16, device=dev)
            ops.linear(x["xq"], x["sx"], x["rs"], ops.B.INTLORA_W_INT16_PLANES, o["planes"], o["sbar"], d, out=Yk,
                       split=o["code"])
            same = same and bool(torch.equal(Yk, g["Y"][:, r0:r0 + d]))
            r0 += d
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in groups] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for s in range(args.steps):
        run(ev[s])
    t1.record(stream)
    torch.cuda.synchronize()
    per_group = []
    for gi, g in enumerate(groups):
        mus = float(np.mean([ev[s][gi][0].elapsed_time(ev[s][gi][1]) for s in range(args.steps)])) * 1e3
        gus = float(np.mean([ev[s][gi][1].elapsed_time(ev[s][gi][2]) for s in range(args.steps)])) * 1e3
        nbytes = sum(l["L"].d * l["L"].n * (2 if bool(o["code"].any()) else 1) for l, o in zip(g["mem"], g["outs"]))
        per_group.append(dict(matrices=[l["L"].name for l in g["mem"]], rows=g["D"], merge_us=round(mus, 2),
                              gemm_us=round(gus, 2), gemm_weight_bytes=nbytes,
                              gemm_weight_GBps=round(nbytes / (gus * 1e-6) / 1e9, 1)))
    return dict(ms_per_step=round(t0.elapsed_time(t1) / args.steps, 4), outputs_equal_per_matrix_calls=same,
                gemm_us_per_step=round(sum(p["gemm_us"] for p in per_group), 1), per_group=per_group,
                note="projections reading the same activations merged into row slices of one buffer and run as "
                     "one linear-layer call; activations of the group's first matrix")


def sweep_measure(args, ops, B, synth, torch, dev, stream):
    """The merge-only sweep of the Llama-3-8B-shaped workload: the MUL merge (U 8-bit,
    r = 64) of every matrix of `args.sweep_blocks` transformer blocks (7 matrices each,
    6.98 G weights over 32 blocks), each with its own weights, factors and layer id.
    Inputs are set up on the GPU first (untimed); one sweep merges every matrix back to
    back into its own output, so the 21 GB of codes and merged integers stream through
    HBM.  Several sweeps are timed; per-shape figures are medians over the matrices of
    that shape and the sweeps."""
    wl = synth.WORKLOADS[4]
    mode, mbits = wl.modes[0]
    nb = max(1, min(args.sweep_blocks, wl.sweep_layers))
    t0 = time.time()
    mats = []
    ws_bytes = 0
    for blk in range(nb):
        for li, L in enumerate(wl.layers):
            lid = synth.layer_id(wl.index, li, blk)
            Wg = torch.from_numpy(synth.sweep_weight(wl, li, blk)).to(dev)
            st = ops.setup_layer(Wg, wl.w_bits, synth.PHILOX_SEED, lid, synth.ALPHA)
            del Wg
            A, Bm = synth.lora(wl, li, block=blk)
            ws_bytes = max(ws_bytes, B.intlora_workspace_bytes(B.INTLORA_OP_MERGE_MUL, B.desc(L.d, L.n, wl.r,
                                                                                               wl.w_bits)))
            st.pop("sigma", None)
            mats.append(dict(L=L, lid=lid, st=st, Ag=torch.from_numpy(A).to(dev), Bg=torch.from_numpy(Bm).to(dev),
                             out=dict(m=torch.empty((L.d, L.n), dtype=torch.int16, device=dev),
                                      sbar=torch.empty(L.d, dtype=torch.float32, device=dev),
                                      zbar=torch.empty(L.d, dtype=torch.int32, device=dev),
                                      split=torch.empty(L.d, dtype=torch.uint8, device=dev),
                                      sat=torch.zeros(2, dtype=torch.int64, device=dev))))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def one(mt):
        ops.merge_mul(mt["st"], mt["Ag"], mt["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, mt["lid"], ws=ws,
                      out=mt["out"])

    for mt in mats:  # warm-up sweep
        one(mt)
    torch.cuda.synchronize()
    sweeps = 5
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in mats]
          for _ in range(sweeps)]
    tot = []
    for sw in range(sweeps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k, mt in enumerate(mats):
            ev[sw][k][0].record(stream)
            one(mt)
            ev[sw][k][1].record(stream)
        b.record(stream)
        tot.append((a, b))
    torch.cuda.synchronize()
    sweep_ms = float(np.median([a.elapsed_time(b) for a, b in tot]))
    elems = sum(mt["L"].d * mt["L"].n for mt in mats)
    alg = sum(merge_alg_bytes(mt["L"].d, mt["L"].n, wl.r, wl.w_bits, mode) for mt in mats)
    per_shape = []
    for L in wl.layers:
        ks = [k for k, mt in enumerate(mats) if mt["L"] is L]
        us = float(np.median([ev[sw][k][0].elapsed_time(ev[sw][k][1]) for sw in range(sweeps) for k in ks])) * 1e3
        mb = merge_alg_bytes(L.d, L.n, wl.r, wl.w_bits, mode)
        per_shape.append(dict(matrix=L.name, d=L.d, n=L.n, count=len(ks), merge_us_median=round(us, 2),
                              alg_GBps=round(mb / (us * 1e-6) / 1e9, 1),
                              pct_hbm_peak=round(100 * mb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
                              G_weights_per_s=round(L.d * L.n / (us * 1e-6) / 1e9, 1)))
    sat = int(sum(int(mt["out"]["sat"][0].item()) for mt in mats))
    del mats, ws
    torch.cuda.empty_cache()
    return dict(blocks=nb, matrices=nb * len(wl.layers), weights=elems, sweeps_timed=sweeps,
                sweep_ms_median=round(sweep_ms, 3), alg_GBps=round(alg / (sweep_ms * 1e-3) / 1e9, 1),
                pct_hbm_peak=round(100 * alg / (sweep_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                G_weights_per_s=round(elems / (sweep_ms * 1e-3) / 1e9, 1), saturated=sat,
                setup_s=round(setup_s, 1), per_shape=per_shape,
                inputs="W per matrix drawn by synth.sweep_weight (row chunks seeded per block and matrix), "
                       "set up on the GPU; layer id 7 * block + matrix")


def stage(name):
    """Names the part of the run that starts next (stderr, flushed), so that a run that
    ends abnormally shows where."""
    sys.stderr.write("[bench] %s\n" % name)
    sys.stderr.flush()


def main():
    args = parse()
    import faulthandler

    faulthandler.enable()  # a fatal signal prints the Python stack of every thread to stderr
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus %d is not supported (the merge "
                                   "would shard by rows and the GEMM by columns, with no exchange between GPUs)"
                                   % args.gpus}))
        sys.exit(2)

    import torch

    from integer_rank_adaptation_amd import binding as B
    from integer_rank_adaptation_amd import ops, synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    B.lib()  # fail loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = synth.WORKLOADS[args.workload]
    M = args.tokens or wl.tokens[0]
    if not 0 <= args.mode_index < len(wl.modes):
        sys.exit("workload %d has %d merge mode(s)" % (args.workload, len(wl.modes)))
    mode, mbits = wl.modes[args.mode_index]

    # ---------------------------------------------------------------- inputs (untimed)
    stage("setup (inputs, set-up kernels)")
    t_setup = time.time()
    layers = []
    ws_bytes = 0
    for li, L in enumerate(wl.layers):
        W = synth.weight(wl, li)
        A, Bm = synth.lora(wl, li)
        X = synth.activations(wl, L.n, M, li)
        lid = synth.layer_id(wl.index, li)
        Wg = torch.from_numpy(W).to(dev)
        st = ops.setup_layer(Wg, wl.w_bits, synth.PHILOX_SEED, lid, synth.ALPHA)
        del Wg
        xq, sx, rs = ops.quant_act(torch.from_numpy(X).to(dev))
        op = B.INTLORA_OP_MERGE_MUL if mode == "mul" else B.INTLORA_OP_MERGE_SHIFT
        ws_bytes = max(ws_bytes, B.intlora_workspace_bytes(op, B.desc(L.d, L.n, wl.r, wl.w_bits)))
        layers.append(dict(L=L, li=li, lid=lid, W=W, A=A, B=Bm, X=X, st=st, Ag=torch.from_numpy(A).to(dev),
                           Bg=torch.from_numpy(Bm).to(dev), xq=xq, sx=sx, rs=rs))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    planes = mode == "mul" and not args.int16_layout and all(L.n % 16 == 0 for L in wl.layers)
    for lay in layers:
        L = lay["L"]
        if planes:
            lay["out"] = dict(planes=torch.empty((L.d, 2 * L.n), dtype=torch.uint8, device=dev),
                              sbar=torch.empty(L.d, dtype=torch.float32, device=dev),
                              zbar=torch.empty(L.d, dtype=torch.int32, device=dev),
                              code=torch.empty(L.d, dtype=torch.uint8, device=dev),
                              sat=torch.zeros(2, dtype=torch.int64, device=dev))
            lay["wfmt"] = B.INTLORA_W_INT16_PLANES
        elif mode == "mul":
            lay["out"] = dict(m=torch.empty((L.d, L.n), dtype=torch.int16, device=dev),
                              sbar=torch.empty(L.d, dtype=torch.float32, device=dev),
                              zbar=torch.empty(L.d, dtype=torch.int32, device=dev),
                              split=torch.empty(L.d, dtype=torch.uint8, device=dev),
                              sat=torch.zeros(2, dtype=torch.int64, device=dev))
            lay["wfmt"] = B.INTLORA_W_INT16
        else:
            lay["out"] = dict(m=torch.empty(ops.code_bytes(L.d, L.n, wl.w_bits), dtype=torch.uint8, device=dev),
                              sbar=torch.empty(L.d, dtype=torch.float32, device=dev),
                              sat=torch.zeros(2, dtype=torch.int64, device=dev))
            lay["wfmt"] = wl.w_bits
        lay["Y"] = torch.empty((M, L.d), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    stream = torch.cuda.current_stream()

    def run_merge(lay):
        if planes:
            ops.merge_mul_planes(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"],
                                 ws=ws, out=lay["out"])
        elif mode == "mul":
            ops.merge_mul(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"], ws=ws,
                          out=lay["out"])
        else:
            ops.merge_shift(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"], ws=ws,
                            out=lay["out"])

    def run_gemm(lay):
        o = lay["out"]
        ops.linear(lay["xq"], lay["sx"], lay["rs"], lay["wfmt"], o["planes"] if planes else o["m"], o["sbar"],
                   lay["L"].d, out=lay["Y"], split=o.get("code") if planes else o.get("split"))

    def step(events=None):
        for k, lay in enumerate(layers):
            if events is not None:
                events[k][0].record(stream)
            run_merge(lay)
            if events is not None:
                events[k][1].record(stream)
            run_gemm(lay)
            if events is not None:
                events[k][2].record(stream)

    def merge_fn(k):
        run_merge(layers[k])

    def gemm_fn(k):
        run_gemm(layers[k])

    stage("timed step (%d warm-up, %d timed)" % (args.warmup, args.steps))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        step(ev[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # ---------------------------------------------------------------- per-kernel medians (untimed region)
    stage("per-kernel medians")
    medians = kernel_medians(args, layers, merge_fn, gemm_fn, torch, dev, stream) if args.kernel_runs > 0 else None
    int16_cmp = None
    if planes and args.kernel_runs > 0:
        int16_cmp = int16_layout_medians(args, layers, ops, synth, wl, mbits, ws, torch, dev, stream)
    lib_cmp = None
    if args.kernel_runs > 0 and not args.no_library_gemm:
        lib_cmp = library_gemm_medians(args, layers, mode, wl.w_bits, planes, torch, stream)

    # ---------------------------------------------------------------- pipelined step (optional)
    stage("pipelined step")
    # The merges run on a side stream, each layer's linear layer waiting only for its own
    # merge; the side stream forks from the step's stream at the start of the step (so a
    # merge never overwrites m while the previous step's linear layer still reads it) and
    # joins it at the end.  The same function is captured in a graph below.
    ms_stream = torch.cuda.Stream()
    done_merge = [torch.cuda.Event() for _ in layers]

    def step_overlap():
        cur = torch.cuda.current_stream()
        ms_stream.wait_stream(cur)
        for k, lay in enumerate(layers):
            with torch.cuda.stream(ms_stream):
                run_merge(lay)
                done_merge[k].record(ms_stream)
            cur.wait_event(done_merge[k])
            run_gemm(lay)
        cur.wait_stream(ms_stream)

    overlap_ms = None
    overlap_same = None
    if not args.no_overlap:
        torch.cuda.synchronize()
        ref_y = [lay["Y"].clone() for lay in layers]
        for lay in layers:
            lay["Y"].zero_()
        for _ in range(args.warmup):
            step_overlap()
        torch.cuda.synchronize()
        overlap_same = all(torch.equal(lay["Y"], r) for lay, r in zip(layers, ref_y))
        del ref_y
        t0_ = torch.cuda.Event(enable_timing=True)
        t1_ = torch.cuda.Event(enable_timing=True)
        t0_.record(stream)
        for _ in range(args.steps):
            step_overlap()
        t1_.record(stream)
        torch.cuda.synchronize()
        overlap_ms = t0_.elapsed_time(t1_) / args.steps

    # ---------------------------------------------------------------- the step as a HIP graph (optional)
    stage("graph replay")
    graph = None
    if not args.no_graph:
        graph = graph_measure(args, layers, step, torch, stream)
        graph_ov = graph_measure(args, layers, step_overlap, torch, stream)
        graph = {"ms_per_step": graph["ms_per_step"], "overlap_ms_per_step": graph_ov["ms_per_step"],
                 "replay_equals_eager": graph["replay_equals_eager"] and graph_ov["replay_equals_eager"]}

    # ---------------------------------------------------------------- QLoRA-style comparison
    ptq = None
    if mode == "mul" and not args.no_ptq:
        stage("QLoRA-style comparison merge")
        ptq = ptq_comparison(args, wl, layers, ws, ops, B, synth, torch, dev, stream)

    fused = None
    if mode == "mul" and max(lay["L"].n for lay in layers) <= 16384 and not args.no_fused:
        stage("fused merge")
        fused = fused_measure(args, wl, layers, ops, synth, torch, dev, stream, mbits)

    codes = None
    if mode == "mul" and wl.w_bits == 4 and mbits <= 4 and not args.no_codes:
        stage("merge keeping the codes + merge-on-load linear layer")
        codes = codes_measure(args, wl, layers, ops, synth, torch, dev, ws, stream, mbits)

    aux_laws = None
    if not args.no_aux_laws:
        stage("auxiliary-matrix laws")
        aux_laws = aux_laws_measure(args, wl, layers, ops, synth, torch, dev, ws, stream, mode, mbits)

    ste = None
    if not args.no_ste:
        stage("straight-through backward")
        ste = ste_measure(args, wl, layers, ops, torch, dev, stream)

    sweep = None
    if not args.no_sweep and M > 32:
        stage("merge sweep over every block")
        sweep = sweep_measure(args, ops, B, synth, torch, dev, stream)

    grouped = None
    if planes and wl.index in SHARED_INPUT_GROUPS and not args.no_grouped:
        stage("shared-input groups")
        grouped = grouped_measure(args, wl, layers, ops, synth, torch, dev, stream, mbits, ws)

    # ---------------------------------------------------------------- per-layer figures
    stage("figures")
    counters = profile_counters(wl.name)
    per_layer = []
    roof_ms = 0.0
    merge_bytes_tot = merge_ms_tot = gemm_ops_tot = gemm_ms_tot = gemm_eops_tot = 0.0
    gemm_bytes_tot = gemm_ops_roof_ms = gemm_bytes_roof_ms = 0.0
    for k, lay in enumerate(layers):
        L = lay["L"]
        mms = float(np.mean([ev[s][k][0].elapsed_time(ev[s][k][1]) for s in range(args.steps)]))
        gms = float(np.mean([ev[s][k][1].elapsed_time(ev[s][k][2]) for s in range(args.steps)]))
        mb = merge_alg_bytes(L.d, L.n, wl.r, wl.w_bits, mode)
        nplanes = planes_multiplied(M, L.d, L.n, bool(lay["out"]["code"].any()), torch) if planes else None
        gops = gemm_exec_ops(M, L.d, L.n, mode, nplanes)
        eops = 2.0 * M * L.d * L.n  # the method's int16 x int8 (or int8 x int8) products, once
        gb = gemm_alg_bytes(M, L.d, L.n, mode, wl.w_bits, nplanes)
        # the linear layer at peak: its products at the int8 rate or its bytes at the HBM
        # rate, whichever takes longer (the bytes, at few tokens or on small layers)
        roof_ms += mb / (HBM_PEAK_GBPS * 1e9) * 1e3 + max(eops / (INT8_PEAK_TOPS * 1e12),
                                                          gb / (HBM_PEAK_GBPS * 1e9)) * 1e3
        gemm_bytes_tot += gb
        gemm_ops_roof_ms += eops / (INT8_PEAK_TOPS * 1e12) * 1e3
        gemm_bytes_roof_ms += gb / (HBM_PEAK_GBPS * 1e9) * 1e3
        merge_bytes_tot += mb
        merge_ms_tot += mms
        gemm_ops_tot += gops
        gemm_eops_tot += eops
        gemm_ms_tot += gms
        row = dict(layer=L.name, d=L.d, n=L.n, merge_us=round(mms * 1e3, 2),
                   merge_alg_GBps=round(mb / (mms * 1e-3) / 1e9, 1),
                   merge_pct_hbm=round(100 * mb / (mms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                   gemm_us=round(gms * 1e3, 2), gemm_exec_TOPS=round(gops / (gms * 1e-3) / 1e12, 1),
                   gemm_exec_pct_int8_peak=round(100 * gops / (gms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
                   gemm_effective_TOPS=round(eops / (gms * 1e-3) / 1e12, 1),
                   gemm_effective_pct_int8_peak=round(100 * eops / (gms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
                   gemm_alg_GBps=round(gb / (gms * 1e-3) / 1e9, 1),
                   sat=int(lay["out"]["sat"][0].item()),
                   int16_split=("balanced" if not bool(lay["out"]["split"].any()) else "bias")
                   if "split" in lay["out"] else None)
        if planes:
            c = lay["out"]["code"]
            row.update(storage="byte planes", gemm_planes_multiplied=nplanes,
                       plane_code_rows={"0_high_plane_zero": int((c == 0).sum()), "1_balanced": int((c == 1).sum()),
                                        "3_bias": int((c == 3).sum())})
            if int16_cmp is not None:
                row.update(gemm_int16_layout_us_median=int16_cmp[k],
                           gemm_int16_layout_exec_TOPS=round(gemm_exec_ops(M, L.d, L.n, mode) /
                                                             (int16_cmp[k] * 1e-6) / 1e12, 1))
        if lib_cmp is not None and lib_cmp[k] is not None:
            row.update(library_int8_gemm_us_median=lib_cmp[k],
                       library_int8_gemm_TOPS=round(2.0 * M * L.d * L.n / (lib_cmp[k] * 1e-6) / 1e12, 1))
        if medians is not None:
            md = medians[k]
            row.update(merge_warm_us_median=md["merge_warm_us"], merge_cold_us_median=md["merge_cold_us"],
                       merge_cold_alg_GBps=round(mb / (md["merge_cold_us"] * 1e-6) / 1e9, 1),
                       gemm_us_median=md["gemm_us"],
                       gemm_exec_TOPS_median=round(gops / (md["gemm_us"] * 1e-6) / 1e12, 1))
        if counters is not None:
            row["counters"] = counters["per_layer"].get(L.name)
        per_layer.append(row)
    # The step's time is that of the fastest measured schedule of the same kernels whose
    # outputs were checked equal to the sequential step's: sequential, pipelined (merges
    # on a second stream), and each replayed from a HIP graph.
    schedules = {"sequential": ms_per_step}
    if overlap_ms is not None and overlap_same:
        schedules["pipelined"] = overlap_ms
    if graph is not None and graph["replay_equals_eager"]:
        schedules["sequential_graph"] = graph["ms_per_step"]
        schedules["pipelined_graph"] = graph["overlap_ms_per_step"]
    schedule = min(schedules, key=schedules.get)
    seq_ms_per_step = ms_per_step
    ms_per_step = schedules[schedule]
    value = 100.0 * roof_ms / ms_per_step
    gemm_avg_ms = gemm_ms_tot / len(layers)
    skinny = M <= 32
    # The dominant kernel's bound: its products (MFMA) or, at few tokens or on layers too
    # small to keep the matrix cores busy, its bytes (HBM).
    gemm_hbm = gemm_bytes_roof_ms > gemm_ops_roof_ms
    if gemm_hbm:
        achieved, peak, runit = gemm_bytes_tot / len(layers) / (gemm_avg_ms * 1e-3) / 1e9, HBM_PEAK_GBPS, "GB/s"
    else:
        achieved, peak, runit = gemm_ops_tot / len(layers) / (gemm_avg_ms * 1e-3) / 1e12, INT8_PEAK_TOPS, "TOP/s"
    if planes:
        kname = ("k_linear_skinny_planes (weight streaming" if skinny else
                 "k_linear_planes (int8 MFMA") + " on the byte-plane storage; planes multiplied per layer: %s)" % [
                     r.get("gemm_planes_multiplied") for r in per_layer]
        kprefix = "k_linear_skinny_planes" if skinny else "k_linear_planes"
    else:
        kname = ("k_linear_skinny (weight streaming, %s)" if skinny else "k_linear (int8 MFMA, %s)") % (
            "int16 two-plane" if mode == "mul" else "int%d" % wl.w_bits)
        kprefix = "k_linear_skinny" if skinny else "k_linear"
    # counter bytes exist for the token count the profiles were taken at (the workload's own)
    traffic = traffic_from_profile(wl.name, kprefix) if M == wl.tokens[0] else None

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "% of MI355X peak (step time at 8 TB/s HBM for the merge's algorithmic bytes + the GEMM at "
                "5.0 POP/s int8 for its products counted once or at 8 TB/s for its bytes, whichever is longer, "
                "over measured step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "schedule": schedule,
        "schedules_ms_per_step": {k: round(v, 4) for k, v in schedules.items()},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": [f"{L.name} {L.d}x{L.n}" for L in wl.layers], "tokens": M,
                   "rank": wl.r, "w_bits": wl.w_bits, "mode": mode, "adapt_bits": mbits},
        "roofline": {"bound": "hbm" if gemm_hbm else "mfma", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": peak, "unit": runit,
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "merge": {"alg_GBps": round(merge_bytes_tot / (merge_ms_tot * 1e-3) / 1e9, 1),
                  "pct_hbm_peak": round(100 * merge_bytes_tot / (merge_ms_tot * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                  "us_per_step": round(merge_ms_tot * 1e3, 1), "bound": "alu (Philox, the Laplace ln and the division per element in the adaptation kernel)"},
        "gemm": {"alg_GBps": round(gemm_bytes_tot / (gemm_ms_tot * 1e-3) / 1e9, 1),
                 "exec_TOPS": round(gemm_ops_tot / (gemm_ms_tot * 1e-3) / 1e12, 1),
                 "exec_frac_int8_peak": round(gemm_ops_tot / (gemm_ms_tot * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                 "effective_TOPS": round(gemm_eops_tot / (gemm_ms_tot * 1e-3) / 1e12, 1),
                 "effective_frac_int8_peak": round(gemm_eops_tot / (gemm_ms_tot * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                 "exec_vs_effective": "exec counts the int8 MFMA operations run (MUL: two byte planes per merged "
                                      "integer, or only the low plane when the merge certified every high byte "
                                      "zero); effective counts each merged-integer x activation product once",
                 "us_per_step": round(gemm_ms_tot * 1e3, 1),
                 "library_int8_gemm_us_sum": round(sum(lib_cmp), 1)
                 if lib_cmp is not None and all(v is not None for v in lib_cmp) else None,
                 "library_int8_gemm_note": "context only: torch._int_mm (the vendor library's int8 GEMM, int32 "
                                           "accumulators, no dequant epilogue or bf16 output) on the same int8 "
                                           "operands, sum of per-layer medians; compare with the sum of "
                                           "per_layer[].gemm_us_median"},
        "kernel_timing": {"runs": args.kernel_runs, "statistic": "median",
                          "cold": "a %d MiB buffer written through HBM before each cold merge run" % args.flush_mib}
        if medians is not None else None,
        "counters": {k: counters[k] for k in ("command", "calibration", "roofline_merge", "roofline_adapt")
                     if k in counters} if counters is not None else None,
        "per_layer": per_layer,
        "overlap_ms_per_step": round(overlap_ms, 4) if overlap_ms is not None else None,
        "overlap_equals_sequential": overlap_same,
        "graph": graph,
        "ptq_comparison": ptq,
        "merge_fused": fused,
        "merge_on_load": codes,
        "ste_backward": ste,
        "aux_laws": aux_laws,
        "sweep": sweep,
        "grouped_shared_inputs": grouped,
        "setup_s": round(setup_s, 1),
    }
    if counters is not None:
        for key in ("roofline_merge", "roofline_adapt"):
            if key in counters:
                result[key] = counters[key]

    # ---------------------------------------------------------------- CPU baseline (oracle)
    stage("CPU baseline (oracle)")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, layers, M, mode, mbits, roof_ms, args.cpu_sample)
    line = json.dumps(result)
    print(line)
    if args.json_out:
        with open(args.json_out, "w") as fh:
            fh.write(line + "\n")


def graph_measure(args, layers, step, torch, stream):
    """The same step captured once in a HIP graph and replayed: the library launches
    only kernels (no memset, copy or allocation), so the whole step captures. Each
    timed replay's outputs are checked against the eager step's before timing."""
    torch.cuda.synchronize()
    ref = [lay["Y"].clone() for lay in layers]
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step()
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    for lay in layers:
        lay["Y"].zero_()
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(lay["Y"], r) for lay, r in zip(layers, ref))
    for _ in range(args.warmup):
        g.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    del g
    return {"ms_per_step": round(ms, 4), "replay_equals_eager": bool(same)}


def cpu_baseline(wl, layers, M, mode, mbits, roof_ms, frac):
    """The oracle, untuned, on a bounded sample of the same step: every layer's merge on
    the first `frac` of its rows and the linear layer on the first `frac` of the tokens
    (all outputs).  The sample's wall time is scaled by 1/frac to a full step."""
    import oracle
    from integer_rank_adaptation_amd import synth

    threads = oracle.num_threads()
    if frac <= 0.0:
        frac = 1.0 / 3.0
    osts = [oracle.setup_layer(lay["W"], synth.PHILOX_SEED, lay["lid"], wl.w_bits, synth.ALPHA)
            for lay in layers]  # the oracle's own stored state (untimed)

    def step_time(fr):
        """Oracle time of the step's merges on the first `fr` of each layer's rows and its
        linear layers on the first `fr` of the tokens, scaled to a full step."""
        t_total = 0.0
        for lay, ost in zip(layers, osts):
            L = lay["L"]
            rows = max(1, int(round(L.d * fr)))
            toks = max(1, int(round(M * fr)))
            xq, sx, _ = oracle.quant_act(lay["X"][:toks])
            t0 = time.perf_counter()
            R = oracle.gen_r_rows(0, rows, L.n, synth.PHILOX_SEED, lay["lid"], ost["c"][:rows])
            if mode == "mul":
                ref = oracle.merge_mul(ost["wround"][:rows], ost["z"][:rows], ost["s"][:rows], R, lay["A"][:rows],
                                       lay["B"], mbits)
            else:
                ref = oracle.merge_shift(ost["wround"][:rows], ost["z"][:rows], ost["s"][:rows], R, lay["A"][:rows],
                                         lay["B"], wl.w_bits, mbits)
            t1 = time.perf_counter()
            # the linear layer over all outputs needs every merged row: the sampled rows'
            # merged integers tiled to d rows (the same cost as the true d x n product)
            m_full = np.resize(ref["m"].astype(np.int32), (L.d, L.n))
            sbar_full = np.resize(ref["sbar"], L.d)
            t2 = time.perf_counter()
            oracle.linear(xq, sx, m_full, sbar_full, want_exact=False)
            t3 = time.perf_counter()
            t_total += (t1 - t0) * (L.d / rows) + (t3 - t2) * (M / toks)
        return t_total

    t_total = step_time(frac)
    repeats = 1
    if t_total < 2.0:  # small workloads: best of 3
        t_total = min([t_total] + [step_time(frac) for _ in range(2)])
        repeats = 3
    frac1 = frac if t_total < 2.0 else frac / 16.0
    oracle.set_threads(1)
    try:
        t_single = step_time(frac1)
    finally:
        oracle.set_threads(threads)
    value = 100.0 * roof_ms / (t_total * 1e3)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(value, 6), "unit": "% of MI355X peak (same definition; oracle step time)",
            "cores": threads, "kind": "oracle",
            "sample": "fraction %.4g of every layer's rows (merge) and tokens (linear), scaled to a full step "
                      "(%.1f s per full step on %d threads)" % (frac, t_total, threads),
            "sample_fraction": round(frac, 6), "repeats": repeats,
            "step_s": round(t_total, 2),
            "single_thread_step_s": round(t_single, 2), "single_thread_sample_fraction": round(frac1, 6),
            "cpu_model": model, "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
            "next_rows_s_per_step": cpu_next_rows(wl, layers, M, mode, mbits, t_total)}


def cpu_next_rows(wl, layers, M, mode, mbits, merge_linear_s, frac=0.02):
    """The oracle of each path beyond the main step, untuned, on the first `frac` of each
    layer's rows (tokens for the linear layer), scaled to a full step: the QLoRA-style
    comparison path (f4), the straight-through backward (f3, binary64), the merge-on-load
    linear layer (f2: merged integers formed from codes + the linear layer).  The fused
    merge (f1) has the same oracle as the MUL merge."""
    import oracle
    from oracle import algebra
    from integer_rank_adaptation_amd import synth

    out = {"f1_fused_merge": "same oracle as the MUL merge (part of step_s)"}
    t_ptq = t_ste = t_codes = 0.0
    for lay in layers:
        L = lay["L"]
        ost = oracle.setup_layer(lay["W"], synth.PHILOX_SEED, lay["lid"], wl.w_bits, synth.ALPHA)
        rows = max(1, int(round(L.d * frac)))
        R = oracle.gen_r_rows(0, rows, L.n, synth.PHILOX_SEED, lay["lid"], ost["c"][:rows])
        t0 = time.perf_counter()
        oracle.ptq_merge(ost["wround"][:rows], ost["z"][:rows], ost["s"][:rows], R, lay["A"][:rows], lay["B"],
                         wl.w_bits)
        t_ptq += (time.perf_counter() - t0) * (L.d / rows)
        G = synth.random_matrix(900 + lay["li"], (rows, L.n), 1e-3)
        t0 = time.perf_counter()
        algebra.ste_backward(ost["wround"][:rows], ost["z"][:rows], lay["A"][:rows], lay["B"], G)
        t_ste += (time.perf_counter() - t0) * (L.d / rows)
        if mode == "mul" and wl.w_bits == 4 and mbits <= 4:
            ref = oracle.merge_mul(ost["wround"][:rows], ost["z"][:rows], ost["s"][:rows], R, lay["A"][:rows],
                                   lay["B"], mbits)
            toks = max(1, int(round(M * frac)))
            xq, sx, _ = oracle.quant_act(lay["X"][:toks])
            ur = np.resize(ref["uround"], (L.d, L.n))
            zb = np.resize(ref["zbar"], L.d)
            sb = np.resize(ref["sbar"], L.d)
            t0 = time.perf_counter()
            m = oracle.merged_from_codes(ur, ost["wround"], ost["z"], zb)
            t1 = time.perf_counter()
            oracle.linear(xq, sx, m, sb, want_exact=False)
            t2 = time.perf_counter()
            t_codes += (t1 - t0) + (t2 - t1) * (M / toks)
    # the other auxiliary laws: R generation under each law on the same rows (the merge
    # after it is the Laplace merge's oracle, part of step_s)
    for dist, name in AUX_LAW_NAMES.items():
        t = 0.0
        for lay in layers:
            L = lay["L"]
            rows = max(1, int(round(L.d * frac)))
            c = np.ones(rows, np.float32)
            t0 = time.perf_counter()
            oracle.gen_r_rows(0, rows, L.n, synth.PHILOX_SEED, lay["lid"], c, dist)
            t += (time.perf_counter() - t0) * (L.d / rows)
        out["f4_aux_law_r_generation_" + name] = round(t, 3)
    out["f4_ptq_merge"] = round(t_ptq, 3)
    out["f3_ste_backward"] = round(t_ste, 3)
    if t_codes > 0.0:
        out["f2_merge_on_load_linear"] = round(t_codes, 3)
    out["sample"] = "first %.3g of each layer's rows (and tokens), scaled to a full step" % frac
    return out


if __name__ == "__main__":
    main()
