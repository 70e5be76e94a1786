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
step's time at MI355X peak (merge algorithmic bytes at 8 TB/s HBM plus the GEMM's
executed int8 MFMA operations at 5.0 POP/s) and T_step the measured time of one step.
Per-layer merge GB/s and GEMM TOP/s are listed alongside.
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


def gemm_exec_ops(M, d, n, mode):
    passes = 2 if mode == "mul" else 1
    return 2.0 * M * d * n * passes


def traffic_from_profile(workload_name):
    """HBM bytes per GEMM launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", workload_name + "_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    from integer_rank_adaptation_amd.profiling import kernel_source_sha

    if rec.get("kernel_source_sha") != kernel_source_sha() or rec.get("workload") != workload_name:
        return None
    return rec.get("hbm_bytes_per_launch")


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
        m = lay["out"]["m"][rows].double()
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
                        same_m_as_three_kernel_merge=bool(torch.equal(outs[k]["m"], lay["out"]["m"]))))
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


def main():
    args = parse()
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
    mode, mbits = wl.modes[0]

    # ---------------------------------------------------------------- inputs (untimed)
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
    for lay in layers:
        L = lay["L"]
        if mode == "mul":
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

    def step(events=None):
        for k, lay in enumerate(layers):
            if events is not None:
                events[k][0].record(stream)
            if mode == "mul":
                ops.merge_mul(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"],
                              ws=ws, out=lay["out"])
            else:
                ops.merge_shift(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"],
                                ws=ws, out=lay["out"])
            if events is not None:
                events[k][1].record(stream)
            ops.linear(lay["xq"], lay["sx"], lay["rs"], lay["wfmt"], lay["out"]["m"], lay["out"]["sbar"], lay["L"].d,
                       out=lay["Y"], split=lay["out"].get("split"))
            if events is not None:
                events[k][2].record(stream)

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

    # ---------------------------------------------------------------- pipelined step (optional)
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
                if mode == "mul":
                    ops.merge_mul(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED, lay["lid"],
                                  ws=ws, out=lay["out"])
                else:
                    ops.merge_shift(lay["st"], lay["Ag"], lay["Bg"], wl.w_bits, mbits, synth.PHILOX_SEED,
                                    lay["lid"], ws=ws, out=lay["out"])
                done_merge[k].record(ms_stream)
            cur.wait_event(done_merge[k])
            ops.linear(lay["xq"], lay["sx"], lay["rs"], lay["wfmt"], lay["out"]["m"], lay["out"]["sbar"],
                       lay["L"].d, out=lay["Y"], split=lay["out"].get("split"))
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
    graph = None
    if not args.no_graph:
        graph = graph_measure(args, layers, step, torch, stream)
        graph_ov = graph_measure(args, layers, step_overlap, torch, stream)
        graph = {"ms_per_step": graph["ms_per_step"], "overlap_ms_per_step": graph_ov["ms_per_step"],
                 "replay_equals_eager": graph["replay_equals_eager"] and graph_ov["replay_equals_eager"]}

    # ---------------------------------------------------------------- QLoRA-style comparison
    ptq = None
    if mode == "mul" and not args.no_ptq:
        ptq = ptq_comparison(args, wl, layers, ws, ops, B, synth, torch, dev, stream)

    fused = None
    if mode == "mul" and max(lay["L"].n for lay in layers) <= 16384 and not args.no_fused:
        fused = fused_measure(args, wl, layers, ops, synth, torch, dev, stream, mbits)

    codes = None
    if mode == "mul" and wl.w_bits == 4 and mbits <= 4 and not args.no_codes:
        codes = codes_measure(args, wl, layers, ops, synth, torch, dev, ws, stream, mbits)

    aux_laws = None
    if not args.no_aux_laws:
        aux_laws = aux_laws_measure(args, wl, layers, ops, synth, torch, dev, ws, stream, mode, mbits)

    ste = None
    if not args.no_ste:
        ste = ste_measure(args, wl, layers, ops, torch, dev, stream)

    # ---------------------------------------------------------------- per-layer figures
    per_layer = []
    roof_ms = 0.0
    merge_bytes_tot = merge_ms_tot = gemm_ops_tot = gemm_ms_tot = 0.0
    for k, lay in enumerate(layers):
        L = lay["L"]
        mms = float(np.mean([ev[s][k][0].elapsed_time(ev[s][k][1]) for s in range(args.steps)]))
        gms = float(np.mean([ev[s][k][1].elapsed_time(ev[s][k][2]) for s in range(args.steps)]))
        mb = merge_alg_bytes(L.d, L.n, wl.r, wl.w_bits, mode)
        gops = gemm_exec_ops(M, L.d, L.n, mode)
        roof_ms += mb / (HBM_PEAK_GBPS * 1e9) * 1e3 + gops / (INT8_PEAK_TOPS * 1e12) * 1e3
        merge_bytes_tot += mb
        merge_ms_tot += mms
        gemm_ops_tot += gops
        gemm_ms_tot += gms
        per_layer.append(dict(layer=L.name, d=L.d, n=L.n, merge_us=round(mms * 1e3, 2),
                              merge_alg_GBps=round(mb / (mms * 1e-3) / 1e9, 1),
                              merge_pct_hbm=round(100 * mb / (mms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                              gemm_us=round(gms * 1e3, 2), gemm_TOPS=round(gops / (gms * 1e-3) / 1e12, 1),
                              gemm_pct_int8_peak=round(100 * gops / (gms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2),
                              sat=int(lay["out"]["sat"][0].item()),
                              int16_split=("balanced" if not bool(lay["out"]["split"].any()) else "bias")
                              if "split" in lay["out"] else None))
    value = 100.0 * roof_ms / ms_per_step
    gemm_avg_ms = gemm_ms_tot / len(layers)
    achieved = gemm_ops_tot / len(layers) / (gemm_avg_ms * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "% of MI355X peak (step time at 8 TB/s HBM for merge bytes + 5.0 POP/s int8 for GEMM ops, "
                "over measured step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": [f"{L.name} {L.d}x{L.n}" for L in wl.layers], "tokens": M,
                   "rank": wl.r, "w_bits": wl.w_bits, "mode": mode, "adapt_bits": mbits},
        "roofline": {"bound": "mfma", "kernel": "k_linear (int8 MFMA, %s)" % ("int16 two-plane" if mode == "mul"
                                                                            else "int%d" % wl.w_bits),
                     "achieved": round(achieved, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(achieved / INT8_PEAK_TOPS, 4), "traffic": traffic_from_profile(wl.name)},
        "merge": {"alg_GBps": round(merge_bytes_tot / (merge_ms_tot * 1e-3) / 1e9, 1),
                  "pct_hbm_peak": round(100 * merge_bytes_tot / (merge_ms_tot * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                  "us_per_step": round(merge_ms_tot * 1e3, 1), "bound": "alu (Philox, the Laplace ln and the division per element in the adaptation kernel)"},
        "gemm": {"exec_TOPS": round(gemm_ops_tot / (gemm_ms_tot * 1e-3) / 1e12, 1),
                 "effective_TOPS": round(gemm_ops_tot / (2 if mode == "mul" else 1) / (gemm_ms_tot * 1e-3) / 1e12, 1),
                 "us_per_step": round(gemm_ms_tot * 1e3, 1)},
        "per_layer": per_layer,
        "overlap_ms_per_step": round(overlap_ms, 4) if overlap_ms is not None else None,
        "overlap_equals_sequential": overlap_same,
        "graph": graph,
        "ptq_comparison": ptq,
        "merge_fused": fused,
        "merge_on_load": codes,
        "ste_backward": ste,
        "aux_laws": aux_laws,
        "setup_s": round(setup_s, 1),
    }

    # ---------------------------------------------------------------- CPU baseline (oracle)
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
    t_total = 0.0
    for lay in layers:
        L = lay["L"]
        # stored state of the oracle's own set-up (untimed)
        ost = oracle.setup_layer(lay["W"], synth.PHILOX_SEED, lay["lid"], wl.w_bits, synth.ALPHA)
        rows = max(1, int(round(L.d * frac)))
        toks = max(1, int(round(M * frac)))
        xq, sx, _ = oracle.quant_act(lay["X"][:toks])
        t0 = time.perf_counter()
        R = oracle.gen_r_rows(0, rows, L.n, synth.PHILOX_SEED, lay["lid"], ost["c"][:rows])
        if mode == "mul":
            ref = oracle.merge_mul(ost["wround"][:rows], ost["z"][:rows], ost["s"][:rows], R, lay["A"][:rows], lay["B"],
                                   mbits)
        else:
            ref = oracle.merge_shift(ost["wround"][:rows], ost["z"][:rows], ost["s"][:rows], R, lay["A"][:rows],
                                     lay["B"], wl.w_bits, mbits)
        t1 = time.perf_counter()
        # the linear layer over all outputs needs every merged row: use the sampled rows'
        # merged integers tiled to d rows (same cost as the true d x n product)
        m_full = np.resize(ref["m"].astype(np.int32), (L.d, L.n))
        sbar_full = np.resize(ref["sbar"], L.d)
        t2 = time.perf_counter()
        oracle.linear(xq, sx, m_full, sbar_full, want_exact=False)
        t3 = time.perf_counter()
        t_total += (t1 - t0) * (L.d / rows) + (t3 - t2) * (M / toks)
    value = 100.0 * roof_ms / (t_total * 1e3)
    return {"value": round(value, 6), "unit": "% of MI355X peak (same definition; oracle step time)",
            "cores": threads, "kind": "oracle",
            "sample": "every layer: merge of the first %.4g of rows, linear on the first %.4g of tokens; "
                      "scaled to a full step (%.1f s per full step)" % (frac, frac, t_total),
            "step_s": round(t_total, 2),
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
