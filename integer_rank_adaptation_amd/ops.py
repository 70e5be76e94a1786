"""Convenience calls over the C ABI: allocate outputs / workspaces with torch (device
memory only) and run one IntLoRA step through libintlora.so.  No arithmetic of the
method happens here."""
from __future__ import annotations

import torch

from . import binding as B


def _dev(t):
    return t.device


def gen_r(d, n, seed, layer_id, c, aux_dist=0):
    out = torch.empty((d, n), dtype=torch.float32, device=_dev(c))
    B.intlora_gen_r(B.desc(d, n, 1, 8, seed, layer_id, aux_dist), c, out)
    return out


def sigma_w(W):
    d, n = W.shape
    out = torch.empty(d, dtype=torch.float32, device=_dev(W))
    B.intlora_stats(B.desc(d, n, 1, 8), B.INTLORA_SIGMA_W, W=W, out0=out)
    return out


def vmc_scale(sigma, alpha, aux_dist=0):
    c = torch.empty_like(sigma)
    if aux_dist == 0:
        B.intlora_vmc_scale(sigma.numel(), sigma, alpha, c)
    else:
        B.intlora_vmc_scale_dist(sigma.numel(), sigma, alpha, aux_dist, c)
    return c


def code_bytes(d, n, w_bits):
    return (d, n) if w_bits == 8 else (d, n // 2)


def base_quant(W, c, w_bits, seed, layer_id, aux_dist=0):
    d, n = W.shape
    wr = torch.empty(code_bytes(d, n, w_bits), dtype=torch.uint8, device=_dev(W))
    z = torch.empty(d, dtype=torch.int32, device=_dev(W))
    s = torch.empty(d, dtype=torch.float32, device=_dev(W))
    B.intlora_base_quant(B.desc(d, n, 1, w_bits, seed, layer_id, aux_dist), W, c, wr, z, s)
    return wr, z, s


def setup_layer(W, w_bits, seed, layer_id, alpha=1.5, aux_dist=0):
    """AQS + VMC set-up of a pretrained layer on the GPU: sigma_W, c, Q[W - R*].  The
    auxiliary law (aux_dist) is kept with the state and used by every merge of it."""
    sig = sigma_w(W)
    c = vmc_scale(sig, alpha, aux_dist)
    wr, z, s = base_quant(W, c, w_bits, seed, layer_id, aux_dist)
    return dict(sigma=sig, c=c, wround=wr, z=z, s=s, aux_dist=aux_dist)


def workspace(op, d, n, r, w_bits, device):
    nbytes = B.intlora_workspace_bytes(op, B.desc(d, n, r, w_bits))
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def u_minmax(st, A, Bm, w_bits, seed, layer_id, ws=None):
    d, r = A.shape
    n = Bm.shape[1]
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    ws = workspace(B.INTLORA_OP_STATS_UMINMAX, d, n, r, w_bits, A.device) if ws is None else ws
    umin = torch.empty(d, dtype=torch.float32, device=A.device)
    umax = torch.empty_like(umin)
    B.intlora_stats(dsc, B.INTLORA_U_MINMAX, None, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm),
                    umin, umax, ws)
    return umin, umax


def merge_mul(st, A, Bm, w_bits, u_bits, seed, layer_id, dbg=False, ws=None, out=None, u_range=None):
    """u_range: optional (u_min, u_max) device tensors [d] used in place of the row range."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    ws = workspace(B.INTLORA_OP_MERGE_MUL, d, n, r, w_bits, dev) if ws is None else ws
    o = out or dict(m=torch.empty((d, n), dtype=torch.int16, device=dev),
                    sbar=torch.empty(d, dtype=torch.float32, device=dev),
                    zbar=torch.empty(d, dtype=torch.int32, device=dev),
                    split=torch.empty(d, dtype=torch.uint8, device=dev),
                    sat=torch.zeros(2, dtype=torch.int64, device=dev))
    if dbg and "uround" not in o:
        o["uround"] = torch.empty((d, n), dtype=torch.uint8, device=dev)
    B.intlora_merge_mul(dsc, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm), u_bits, o["m"],
                        o["sbar"], o["zbar"], m_split=o.get("split"), u_round_dbg=o.get("uround") if dbg else None,
                        sat_count=o["sat"], ws=ws, u_min=u_range[0] if u_range else None,
                        u_max=u_range[1] if u_range else None)
    return o


def merge_mul_planes(st, A, Bm, w_bits, u_bits, seed, layer_id, dbg=False, ws=None, out=None, u_range=None):
    """MUL merge writing the merged integers as their two int8 byte planes (d x 2n
    bytes) with per-row plane codes, for the linear layer's INT16_PLANES format."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    ws = workspace(B.INTLORA_OP_MERGE_MUL, d, n, r, w_bits, dev) if ws is None else ws
    o = out or dict(planes=torch.empty((d, 2 * n), dtype=torch.uint8, device=dev),
                    sbar=torch.empty(d, dtype=torch.float32, device=dev),
                    zbar=torch.empty(d, dtype=torch.int32, device=dev),
                    code=torch.empty(d, dtype=torch.uint8, device=dev),
                    sat=torch.zeros(2, dtype=torch.int64, device=dev))
    if dbg and "uround" not in o:
        o["uround"] = torch.empty((d, n), dtype=torch.uint8, device=dev)
    B.intlora_merge_mul_planes(dsc, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm), u_bits,
                               o["planes"], o["sbar"], o["zbar"], o["code"],
                               u_round_dbg=o.get("uround") if dbg else None, sat_count=o["sat"], ws=ws,
                               u_min=u_range[0] if u_range else None, u_max=u_range[1] if u_range else None)
    return o


def merge_mul_noalloc(st, A, Bm, w_bits, u_bits, seed, layer_id, dbg=False, out=None, u_range=None):
    """MUL merge with the library's own per-device scratch (no workspace); same outputs
    as merge_mul."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    o = out or dict(m=torch.empty((d, n), dtype=torch.int16, device=dev),
                    sbar=torch.empty(d, dtype=torch.float32, device=dev),
                    zbar=torch.empty(d, dtype=torch.int32, device=dev),
                    split=torch.empty(d, dtype=torch.uint8, device=dev),
                    sat=torch.zeros(2, dtype=torch.int64, device=dev))
    if dbg and "uround" not in o:
        o["uround"] = torch.empty((d, n), dtype=torch.uint8, device=dev)
    B.intlora_merge_mul_noalloc(dsc, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm), u_bits, o["m"],
                                o["sbar"], o["zbar"], m_split=o.get("split"),
                                u_round_dbg=o.get("uround") if dbg else None, sat_count=o["sat"],
                                u_min=u_range[0] if u_range else None, u_max=u_range[1] if u_range else None)
    return o


def merge_mul_fused(st, A, Bm, w_bits, u_bits, seed, layer_id, dbg=False, out=None):
    """Fused single-pass MUL merge (no workspace); same outputs as merge_mul."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    o = out or dict(m=torch.empty((d, n), dtype=torch.int16, device=dev),
                    sbar=torch.empty(d, dtype=torch.float32, device=dev),
                    zbar=torch.empty(d, dtype=torch.int32, device=dev),
                    split=torch.empty(d, dtype=torch.uint8, device=dev),
                    sat=torch.zeros(2, dtype=torch.int64, device=dev))
    if dbg and "uround" not in o:
        o["uround"] = torch.empty((d, n), dtype=torch.uint8, device=dev)
    B.intlora_merge_mul_fused(dsc, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm), u_bits, o["m"],
                              o["sbar"], o["zbar"], m_split=o.get("split"),
                              u_round_dbg=o.get("uround") if dbg else None, sat_count=o["sat"])
    return o


def merge_mul_codes(st, A, Bm, w_bits, u_bits, seed, layer_id, ws=None, out=None):
    """MUL merge keeping U's codes (packed nibbles d x n/2) with s_bar, z_bar, for the
    merge-on-load linear layer."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    ws = workspace(B.INTLORA_OP_MERGE_MUL, d, n, r, w_bits, dev) if ws is None else ws
    o = out or dict(ucode=torch.empty((d, n // 2), dtype=torch.uint8, device=dev),
                    sbar=torch.empty(d, dtype=torch.float32, device=dev),
                    zbar=torch.empty(d, dtype=torch.int32, device=dev))
    B.intlora_merge_mul_codes(dsc, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm), u_bits, o["ucode"],
                              o["sbar"], o["zbar"], ws=ws)
    return o


def merge_shift(st, A, Bm, w_bits, v_bits, seed, layer_id, dbg=False, ws=None, out=None, u_range=None):
    """u_range: optional (u_min, u_max) device tensors [d] used in place of the row range."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    ws = workspace(B.INTLORA_OP_MERGE_SHIFT, d, n, r, w_bits, dev) if ws is None else ws
    o = out or dict(m=torch.empty(code_bytes(d, n, w_bits), dtype=torch.uint8, device=dev),
                    sbar=torch.empty(d, dtype=torch.float32, device=dev),
                    sat=torch.zeros(2, dtype=torch.int64, device=dev))
    if dbg and "shift" not in o:
        o["shift"] = torch.empty((d, n), dtype=torch.uint8, device=dev)
    B.intlora_merge_shift(dsc, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm), v_bits, o["m"],
                          o["sbar"], o.get("shift") if dbg else None, o["sat"], ws,
                          u_min=u_range[0] if u_range else None, u_max=u_range[1] if u_range else None)
    return o


def merge_ptq(st, A, Bm, w_bits, bits, seed, layer_id, ws=None, out=None):
    """QLoRA-style comparison path: x = (s w + R*) + AB, per-row requant at `bits`."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits, seed, layer_id, st.get("aux_dist", 0))
    ws = workspace(B.INTLORA_OP_MERGE_PTQ, d, n, r, w_bits, dev) if ws is None else ws
    o = out or dict(code=torch.empty(code_bytes(d, n, bits), dtype=torch.uint8, device=dev),
                    s=torch.empty(d, dtype=torch.float32, device=dev),
                    z=torch.empty(d, dtype=torch.int32, device=dev))
    B.intlora_merge_ptq(dsc, B.base(st["wround"], st["z"], st["s"], st["c"]), B.lora(A, Bm), bits, o["code"], o["s"],
                        o["z"], ws)
    return o


def ste_backward(st, A, Bm, G, w_bits, ws=None, out=None):
    """Straight-through backward to the LoRA factors: dA = (G.[w != 0]) B^T, dB = A^T (G.[w != 0])."""
    d, r = A.shape
    n = Bm.shape[1]
    dev = A.device
    dsc = B.desc(d, n, r, w_bits)
    if ws is None:
        nb = B.intlora_workspace_bytes(B.INTLORA_OP_STE_BACKWARD, dsc)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    o = out or dict(dA=torch.empty((d, r), dtype=torch.float32, device=dev),
                    dB=torch.empty((r, n), dtype=torch.float32, device=dev))
    B.intlora_ste_backward(dsc, st["wround"], st["z"], A, Bm, G, o["dA"], o["dB"], ws)
    return o


def quant_act(X):
    M, n = X.shape
    xq = torch.empty((M, n), dtype=torch.int8, device=X.device)
    sx = torch.empty(M, dtype=torch.float32, device=X.device)
    rs = torch.empty(M, dtype=torch.int32, device=X.device)
    B.intlora_quant_act(M, n, X, xq, sx, rs)
    return xq, sx, rs


def linear(xq, sx, rowsum, wfmt, m, sbar, d, acc_dbg=False, out=None, split=None):
    """split: the MUL merge's per-row split codes (INT16 only); None = bias split for
    every row."""
    M, n = xq.shape
    Y = torch.empty((M, d), dtype=torch.int16, device=xq.device) if out is None else out
    planes = 2 if wfmt in (B.INTLORA_W_INT16, B.INTLORA_W_INT16_PLANES) else 1
    acc = torch.empty((planes, M, d), dtype=torch.int32, device=xq.device) if acc_dbg else None
    B.intlora_linear_fwd(M, d, n, xq, sx, rowsum, wfmt, m, split, sbar, Y, acc)
    return Y, acc


def linear_codes(xq, sx, ucode, wcode, z, zbar, sbar, d, acc_dbg=False, out=None):
    """Merge-on-load linear layer: m = (U_round - z_bar) (W_round - z) formed in the GEMM
    from the packed 4-bit codes (d x n/2 each)."""
    M, n = xq.shape
    Y = torch.empty((M, d), dtype=torch.int16, device=xq.device) if out is None else out
    acc = torch.empty((2, M, d), dtype=torch.int32, device=xq.device) if acc_dbg else None
    B.intlora_linear_fwd_codes(M, d, n, xq, sx, ucode, wcode, z, zbar, sbar, Y, acc)
    return Y, acc
