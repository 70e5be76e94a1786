"""Thin ctypes binding of libintlora.so (C ABI in include/intlora.h).

Argument marshalling only: every function here has the name of the C entry point it
calls, takes torch tensors (device memory) where the C function takes device pointers,
passes torch's current HIP stream, and raises ``IntLoraError`` on a non-zero status.
There is no fallback: without the compiled library every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libintlora.so")

# status codes / enums (mirror include/intlora.h)
INTLORA_OK, INTLORA_EINVAL, INTLORA_ESHAPE, INTLORA_EALIGN, INTLORA_EWORKSPACE, INTLORA_EDEVICE, INTLORA_ELAUNCH = range(7)
INTLORA_SIGMA_W, INTLORA_U_MINMAX = 0, 1
INTLORA_W_INT4, INTLORA_W_INT8, INTLORA_W_INT16, INTLORA_W_INT16_PLANES = 4, 8, 16, 17
INTLORA_AUX_LAPLACE, INTLORA_AUX_GAUSS, INTLORA_AUX_CAUCHY, INTLORA_AUX_STUDENT_T2 = 0, 1, 2, 3
INTLORA_OP_STATS_UMINMAX, INTLORA_OP_MERGE_MUL, INTLORA_OP_MERGE_SHIFT, INTLORA_OP_LINEAR, INTLORA_OP_BASE_QUANT = 1, 2, 3, 4, 5
INTLORA_OP_MERGE_PTQ, INTLORA_OP_STE_BACKWARD = 6, 7


class IntLoraError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("n", ctypes.c_int64), ("r", ctypes.c_int32), ("w_bits", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("layer_id", ctypes.c_uint32), ("aux_dist", ctypes.c_uint32)]


class Base(ctypes.Structure):
    _fields_ = [("w_round", ctypes.c_void_p), ("z", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("vmc_c", ctypes.c_void_p)]


class Lora(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p)]


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SIG = {
    "intlora_status_string": (ctypes.c_char_p, [_INT]),
    "intlora_last_error": (ctypes.c_char_p, []),
    "intlora_version": (_INT, []),
    "intlora_workspace_bytes": (ctypes.c_size_t, [_INT, ctypes.POINTER(Desc), _I64]),
    "intlora_gen_r": (_INT, [ctypes.POINTER(Desc), _P, _P, _P]),
    "intlora_stats": (_INT, [ctypes.POINTER(Desc), _INT, _P, ctypes.POINTER(Base), ctypes.POINTER(Lora), _P, _P, _P,
                             ctypes.c_size_t, _P]),
    "intlora_vmc_scale": (_INT, [_I64, _P, ctypes.c_double, _P, _P]),
    "intlora_vmc_scale_dist": (_INT, [_I64, _P, ctypes.c_double, ctypes.c_uint32, _P, _P]),
    "intlora_base_quant": (_INT, [ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _P]),
    "intlora_merge_mul": (_INT, [ctypes.POINTER(Desc), ctypes.POINTER(Base), ctypes.POINTER(Lora), _INT, _P, _P, _P,
                                 _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "intlora_merge_mul_planes": (_INT, [ctypes.POINTER(Desc), ctypes.POINTER(Base), ctypes.POINTER(Lora), _INT, _P,
                                        _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "intlora_merge_mul_noalloc": (_INT, [ctypes.POINTER(Desc), ctypes.POINTER(Base), ctypes.POINTER(Lora), _INT, _P,
                                         _P, _P, _P, _P, _P, _P, _P, _P]),
    "intlora_merge_mul_fused": (_INT, [ctypes.POINTER(Desc), ctypes.POINTER(Base), ctypes.POINTER(Lora), _INT, _P,
                                       _P, _P, _P, _P, _P, _P]),
    "intlora_merge_mul_codes": (_INT, [ctypes.POINTER(Desc), ctypes.POINTER(Base), ctypes.POINTER(Lora), _INT, _P,
                                       _P, _P, _P, ctypes.c_size_t, _P]),
    "intlora_merge_shift": (_INT, [ctypes.POINTER(Desc), ctypes.POINTER(Base), ctypes.POINTER(Lora), _INT, _P, _P,
                                   _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "intlora_merge_ptq": (_INT, [ctypes.POINTER(Desc), ctypes.POINTER(Base), ctypes.POINTER(Lora), _INT, _P, _P, _P,
                                 _P, ctypes.c_size_t, _P]),
    "intlora_ste_backward": (_INT, [ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "intlora_quant_act": (_INT, [_I64, _I64, _P, _P, _P, _P, _P]),
    "intlora_linear_fwd": (_INT, [_I64, _I64, _I64, _P, _P, _P, _INT, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "intlora_linear_fwd_codes": (_INT, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "intlora_debug_ln": (_INT, [_I64, _P, _P, _P]),
    "intlora_debug_aux": (_INT, [_I64, _P, ctypes.c_uint32, _P, _P]),
    "intlora_debug_mfma_chain": (_INT, [_INT, _I64, _I64, _INT, _P, _P, _P, _P]),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                               "g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != INTLORA_OK:
        detail = lib().intlora_last_error().decode()
        raise IntLoraError(status, where, detail or lib().intlora_status_string(status).decode())


def desc(d: int, n: int, r: int, w_bits: int, seed: int = 0, layer_id: int = 0, aux_dist: int = 0) -> Desc:
    return Desc(d, n, r, w_bits, seed, layer_id, aux_dist)


def base(w_round, z, s, vmc_c) -> Base:
    return Base(_ptr(w_round), _ptr(z), _ptr(s), _ptr(vmc_c))


def lora(A, B) -> Lora:
    return Lora(_ptr(A), _ptr(B))


def intlora_version() -> int:
    return int(lib().intlora_version())


def intlora_workspace_bytes(op: int, dsc: Desc, M: int = 0) -> int:
    return int(lib().intlora_workspace_bytes(op, ctypes.byref(dsc), M))


def intlora_gen_r(dsc: Desc, vmc_c, r_out, stream=None):
    _check(lib().intlora_gen_r(ctypes.byref(dsc), _ptr(vmc_c), _ptr(r_out), _stream(stream)), "intlora_gen_r")


def intlora_stats(dsc: Desc, mode: int, W=None, bs: Base | None = None, lr: Lora | None = None, out0=None, out1=None,
                  ws=None, stream=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_stats(ctypes.byref(dsc), mode, _ptr(W), ctypes.byref(bs) if bs is not None else None,
                               ctypes.byref(lr) if lr is not None else None, _ptr(out0), _ptr(out1), _ptr(ws), wsb,
                               _stream(stream)), "intlora_stats")


def intlora_vmc_scale(d: int, sigma_w, alpha: float, c_out, stream=None):
    _check(lib().intlora_vmc_scale(d, _ptr(sigma_w), float(alpha), _ptr(c_out), _stream(stream)),
           "intlora_vmc_scale")


def intlora_vmc_scale_dist(d: int, sigma_w, alpha: float, aux_dist: int, c_out, stream=None):
    _check(lib().intlora_vmc_scale_dist(d, _ptr(sigma_w), float(alpha), aux_dist, _ptr(c_out), _stream(stream)),
           "intlora_vmc_scale_dist")


def intlora_base_quant(dsc: Desc, W, vmc_c, w_round_out, z_out, s_out, stream=None):
    _check(lib().intlora_base_quant(ctypes.byref(dsc), _ptr(W), _ptr(vmc_c), _ptr(w_round_out), _ptr(z_out),
                                    _ptr(s_out), _stream(stream)), "intlora_base_quant")


def intlora_merge_mul(dsc: Desc, bs: Base, lr: Lora, u_bits: int, m, s_bar, z_bar, m_split=None, u_round_dbg=None,
                      sat_count=None, ws=None, stream=None, u_min=None, u_max=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_merge_mul(ctypes.byref(dsc), ctypes.byref(bs), ctypes.byref(lr), u_bits, _ptr(u_min),
                                   _ptr(u_max), _ptr(m), _ptr(s_bar), _ptr(z_bar), _ptr(m_split), _ptr(u_round_dbg),
                                   _ptr(sat_count), _ptr(ws), wsb, _stream(stream)), "intlora_merge_mul")


def intlora_merge_mul_planes(dsc: Desc, bs: Base, lr: Lora, u_bits: int, m_planes, s_bar, z_bar, plane_code,
                             u_round_dbg=None, sat_count=None, ws=None, stream=None, u_min=None, u_max=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_merge_mul_planes(ctypes.byref(dsc), ctypes.byref(bs), ctypes.byref(lr), u_bits, _ptr(u_min),
                                          _ptr(u_max), _ptr(m_planes), _ptr(s_bar), _ptr(z_bar), _ptr(plane_code),
                                          _ptr(u_round_dbg), _ptr(sat_count), _ptr(ws), wsb, _stream(stream)),
           "intlora_merge_mul_planes")


def intlora_merge_mul_noalloc(dsc: Desc, bs: Base, lr: Lora, u_bits: int, m, s_bar, z_bar, m_split=None,
                              u_round_dbg=None, sat_count=None, stream=None, u_min=None, u_max=None):
    _check(lib().intlora_merge_mul_noalloc(ctypes.byref(dsc), ctypes.byref(bs), ctypes.byref(lr), u_bits, _ptr(u_min),
                                           _ptr(u_max), _ptr(m), _ptr(s_bar), _ptr(z_bar), _ptr(m_split),
                                           _ptr(u_round_dbg), _ptr(sat_count), _stream(stream)),
           "intlora_merge_mul_noalloc")


def intlora_merge_mul_fused(dsc: Desc, bs: Base, lr: Lora, u_bits: int, m, s_bar, z_bar, m_split=None,
                            u_round_dbg=None, sat_count=None, stream=None):
    _check(lib().intlora_merge_mul_fused(ctypes.byref(dsc), ctypes.byref(bs), ctypes.byref(lr), u_bits, _ptr(m),
                                         _ptr(s_bar), _ptr(z_bar), _ptr(m_split), _ptr(u_round_dbg),
                                         _ptr(sat_count), _stream(stream)), "intlora_merge_mul_fused")


def intlora_merge_mul_codes(dsc: Desc, bs: Base, lr: Lora, u_bits: int, u_code, s_bar, z_bar, ws=None, stream=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_merge_mul_codes(ctypes.byref(dsc), ctypes.byref(bs), ctypes.byref(lr), u_bits, _ptr(u_code),
                                         _ptr(s_bar), _ptr(z_bar), _ptr(ws), wsb, _stream(stream)),
           "intlora_merge_mul_codes")


def intlora_merge_shift(dsc: Desc, bs: Base, lr: Lora, v_bits: int, m, s_bar, shift_dbg=None, sat_count=None, ws=None,
                        stream=None, u_min=None, u_max=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_merge_shift(ctypes.byref(dsc), ctypes.byref(bs), ctypes.byref(lr), v_bits, _ptr(u_min),
                                     _ptr(u_max), _ptr(m), _ptr(s_bar), _ptr(shift_dbg), _ptr(sat_count), _ptr(ws),
                                     wsb, _stream(stream)), "intlora_merge_shift")


def intlora_merge_ptq(dsc: Desc, bs: Base, lr: Lora, bits: int, code, s_out, z_out, ws=None, stream=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_merge_ptq(ctypes.byref(dsc), ctypes.byref(bs), ctypes.byref(lr), bits, _ptr(code),
                                   _ptr(s_out), _ptr(z_out), _ptr(ws), wsb, _stream(stream)), "intlora_merge_ptq")


def intlora_ste_backward(dsc: Desc, w_round, z, A, B, G, dA, dB, ws=None, stream=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_ste_backward(ctypes.byref(dsc), _ptr(w_round), _ptr(z), _ptr(A), _ptr(B), _ptr(G), _ptr(dA),
                                      _ptr(dB), _ptr(ws), wsb, _stream(stream)), "intlora_ste_backward")


def intlora_quant_act(M: int, n: int, X, xq, s_x, x_rowsum=None, stream=None):
    _check(lib().intlora_quant_act(M, n, _ptr(X), _ptr(xq), _ptr(s_x), _ptr(x_rowsum), _stream(stream)),
           "intlora_quant_act")


def intlora_linear_fwd(M: int, d: int, n: int, xq, s_x, x_rowsum, wfmt: int, m, m_split, s_bar, Y_bf16, acc_dbg=None,
                       ws=None, stream=None):
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().intlora_linear_fwd(M, d, n, _ptr(xq), _ptr(s_x), _ptr(x_rowsum), wfmt, _ptr(m), _ptr(m_split),
                                    _ptr(s_bar), _ptr(Y_bf16), _ptr(acc_dbg), _ptr(ws), wsb, _stream(stream)),
           "intlora_linear_fwd")


def intlora_linear_fwd_codes(M: int, d: int, n: int, xq, s_x, u_code, w_round, z, z_bar, s_bar, Y_bf16, acc_dbg=None,
                             stream=None):
    _check(lib().intlora_linear_fwd_codes(M, d, n, _ptr(xq), _ptr(s_x), _ptr(u_code), _ptr(w_round), _ptr(z),
                                          _ptr(z_bar), _ptr(s_bar), _ptr(Y_bf16), _ptr(acc_dbg), _stream(stream)),
           "intlora_linear_fwd_codes")


def intlora_debug_ln(count: int, G, out, stream=None):
    _check(lib().intlora_debug_ln(count, _ptr(G), _ptr(out), _stream(stream)), "intlora_debug_ln")


def intlora_debug_aux(blocks: int, words, aux_dist: int, out, stream=None):
    _check(lib().intlora_debug_aux(blocks, _ptr(words), aux_dist, _ptr(out), _stream(stream)), "intlora_debug_aux")


def intlora_debug_mfma_chain(form: int, d: int, n: int, r: int, A, B, acc, stream=None):
    _check(lib().intlora_debug_mfma_chain(form, d, n, r, _ptr(A), _ptr(B), _ptr(acc), _stream(stream)),
           "intlora_debug_mfma_chain")
