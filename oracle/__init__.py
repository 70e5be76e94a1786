"""CPU oracle for the IntLoRA integer merge and integer linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with the
GPU library (``integer_rank_adaptation_amd``) and never imports it.

The scalar arithmetic lives in ``intlora_oracle.c`` (plain C, compiled with
``-ffp-contract=off``, OpenMP over independent rows/tokens only); this module marshals
numpy arrays into it and adds the binary64 algebra of the pages (``algebra``).

Pins (see ``tests/test_oracle_*.py``): Philox against rocRAND's reference engine,
the binary32 log against 40-digit decimal logarithms on its whole input domain, the
merges against exact rationals, brute force and the closed forms of the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import algebra  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "intlora_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    """Load the compiled oracle (building it only when nothing is built yet)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_F32 = ctypes.c_float
_F64 = ctypes.c_double


def _declare(L):
    sig = {
        "ora_philox4x32_10": (None, [_P, _P, _P]),
        "ora_philox_batch": (None, [_I64, _P, _P, _P]),
        "ora_ln_rn32": (_F32, [_F32]),
        "ora_laplace": (_F32, [_U32]),
        "ora_gen_r": (None, [_I64, _I64, _U64, _U32, _P, _P]),
        "ora_gen_r_rows": (None, [_I64, _I64, _I64, _U64, _U32, _P, _P]),
        "ora_sigma_w": (None, [_I64, _I64, _P, _P]),
        "ora_vmc_scale": (None, [_I64, _P, _F64, _P]),
        "ora_base_quant": (None, [_I64, _I64, _I32, _P, _P, _P, _P, _P]),
        "ora_adaptation": (None, [_I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "ora_mul_params": (None, [_I64, _I32, _P, _P, _P, _P]),
        "ora_merge_mul": (_I64, [_I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32]),
        "ora_log2_round": (_I32, [_F32]),
        "ora_shift_scale": (_F32, [_F32, _F32]),
        "ora_merge_shift": (_I64, [_I64, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32]),
        "ora_ptq_merge": (None, [_I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
        "ora_quant_act": (None, [_I64, _I64, _P, _P, _P, _P]),
        "ora_bf16_rne": (ctypes.c_uint16, [_F32]),
        "ora_linear": (None, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
        "ora_linear_sampled": (None, [_I64, _P, _P, _I64, _P, _P, _P, _P, _P, _P]),
        "ora_num_threads": (_I32, []),
        "ora_set_threads": (None, [_I32]),
        "ora_laplace_batch": (None, [_I64, _P, _P]),
        "ora_ln_batch": (None, [_I64, _P, _P]),
        "ora_log2_round_batch": (None, [_I64, _P, _P]),
        "ora_cospi": (_F64, [_F64]),
        "ora_sinpi": (_F64, [_F64]),
        "ora_tanpi": (_F64, [_F64]),
        "ora_aux": (_F32, [_P, _I32, _I32]),
        "ora_trig_batch": (None, [_I64, _P, _I32, _P]),
        "ora_aux_batch": (None, [_I64, _P, _I32, _P]),
        "ora_gen_r_dist": (None, [_I64, _I64, _I64, _U64, _U32, _I32, _P, _P]),
        "ora_vmc_scale_dist": (None, [_I64, _P, _F64, _I32, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def num_threads() -> int:
    return int(lib().ora_num_threads())


def set_threads(t: int) -> None:
    """Threads of the oracle's row / token loops (t >= 1)."""
    lib().ora_set_threads(int(t))


# --------------------------------------------------------------------------- RNG
def philox(ctr, key):
    """Philox4x32-10 of each (counter[4], key[2]) row -> uint32[N, 4]."""
    ctr = _c(ctr, np.uint32).reshape(-1, 4)
    key = _c(key, np.uint32).reshape(-1, 2)
    assert ctr.shape[0] == key.shape[0]
    out = np.empty_like(ctr)
    lib().ora_philox_batch(ctr.shape[0], _p(ctr), _p(key), _p(out))
    return out


def ln_rn32(g):
    g = _c(g, np.float32)
    out = np.empty_like(g)
    lib().ora_ln_batch(g.size, _p(g), _p(out))
    return out


def laplace(words):
    words = _c(words, np.uint32)
    out = np.empty(words.shape, np.float32)
    lib().ora_laplace_batch(words.size, _p(words), _p(out))
    return out


def gen_r(d, n, seed, layer_id, c, aux_dist=0):
    """R* = c * sample, the sample under law aux_dist (0 Laplace, 1 Gaussian, 2 Cauchy,
    3 Student-t(2); IntLoRA "1. AQS" and the summary table's distribution ablation)."""
    c = _c(c, np.float32)
    assert c.shape == (d,)
    out = np.empty((d, n), np.float32)
    if aux_dist == 0:
        lib().ora_gen_r(d, n, seed, layer_id, _p(c), _p(out))
    else:
        lib().ora_gen_r_dist(0, d, n, seed, layer_id, int(aux_dist), _p(c), _p(out))
    return out


def aux_samples(words, aux_dist):
    """The unscaled sample of every element of the Philox blocks `words` (..., 4)."""
    words = _c(words, np.uint32).reshape(-1, 4)
    out = np.empty(words.shape, np.float32)
    lib().ora_aux_batch(words.shape[0], _p(words), int(aux_dist), _p(out))
    return out


def trig_pi(v, kind):
    """binary64 cos(pi v) (kind 0), sin(pi v) (1) for 0 < v < 2, tan(pi v) (2) for |v| < 1/2,
    v with at most 24 significant bits (the arguments the samplers produce)."""
    v = _c(v, np.float64)
    out = np.empty_like(v)
    lib().ora_trig_batch(v.size, _p(v), int(kind), _p(out))
    return out


def gen_r_rows(row0, rows, n, seed, layer_id, c_rows, aux_dist=0):
    c_rows = _c(c_rows, np.float32)
    assert c_rows.shape == (rows,)
    out = np.empty((rows, n), np.float32)
    if aux_dist == 0:
        lib().ora_gen_r_rows(row0, rows, n, seed, layer_id, _p(c_rows), _p(out))
    else:
        lib().ora_gen_r_dist(row0, rows, n, seed, layer_id, int(aux_dist), _p(c_rows), _p(out))
    return out


# --------------------------------------------------------------------------- setup
def sigma_w(W):
    W = _c(W, np.float32)
    d, n = W.shape
    out = np.empty(d, np.float32)
    lib().ora_sigma_w(d, n, _p(W), _p(out))
    return out


def vmc_scale(sigma, alpha, aux_dist=0):
    """c = RN32((sigma_W / sigma_R)^alpha): sigma_R = sqrt(2) for Laplace(0, 1), 1 for the
    other laws of the auxiliary-matrix ablation (IntLoRA, "3. VMC")."""
    sigma = _c(sigma, np.float32)
    out = np.empty_like(sigma)
    if aux_dist == 0:
        lib().ora_vmc_scale(sigma.size, _p(sigma), float(alpha), _p(out))
    else:
        lib().ora_vmc_scale_dist(sigma.size, _p(sigma), float(alpha), int(aux_dist), _p(out))
    return out


def base_quant(W, rstar, bits):
    W = _c(W, np.float32)
    rstar = _c(rstar, np.float32)
    d, n = W.shape
    wr = np.empty((d, n), np.uint8)
    z = np.empty(d, np.int32)
    s = np.empty(d, np.float32)
    lib().ora_base_quant(d, n, bits, _p(W), _p(rstar), _p(wr), _p(z), _p(s))
    return wr, z, s


def setup_layer(W, seed, layer_id, bits, alpha=1.5, aux_dist=0):
    """AQS + VMC set-up of one pretrained layer: sigma_W -> c -> R* -> Q[W - R*]."""
    d, n = W.shape
    sig = sigma_w(W)
    c = vmc_scale(sig, alpha, aux_dist)
    rstar = gen_r(d, n, seed, layer_id, c, aux_dist)
    wr, z, s = base_quant(W, rstar, bits)
    return dict(sigma=sig, c=c, rstar=rstar, wround=wr, z=z, s=s)


# --------------------------------------------------------------------------- merge
def adaptation(wround, z, s, rstar, A, B, want_u=True):
    wround = _c(wround, np.uint8)
    rows, n = wround.shape
    A = _c(A, np.float32)
    B = _c(B, np.float32)
    r = A.shape[1]
    assert A.shape == (rows, r) and B.shape == (r, n)
    z = _c(z, np.int32)
    s = _c(s, np.float32)
    rstar = _c(rstar, np.float32)
    u = np.empty((rows, n), np.float32) if want_u else None
    umin = np.empty(rows, np.float32)
    umax = np.empty(rows, np.float32)
    lib().ora_adaptation(rows, n, r, _p(wround), _p(z), _p(s), _p(rstar), _p(A), _p(B), _p(u), _p(umin), _p(umax))
    return u, umin, umax


def mul_params(umin, umax, u_bits):
    umin = _c(umin, np.float32)
    umax = _c(umax, np.float32)
    sbar = np.empty_like(umin)
    zbar = np.empty(umin.shape, np.int32)
    lib().ora_mul_params(umin.size, u_bits, _p(umin), _p(umax), _p(sbar), _p(zbar))
    return sbar, zbar


def merge_mul(wround, z, s, rstar, A, B, u_bits, u_range=None):
    """u_range: optional (u_min, u_max) per row, used in place of the row's own range."""
    wround = _c(wround, np.uint8)
    rows, n = wround.shape
    A = _c(A, np.float32)
    B = _c(B, np.float32)
    r = A.shape[1]
    assert A.shape == (rows, r) and B.shape == (r, n)
    z, s, rstar = _c(z, np.int32), _c(s, np.float32), _c(rstar, np.float32)
    m = np.empty((rows, n), np.int16)
    ur = np.empty((rows, n), np.uint8)
    sbar = np.empty(rows, np.float32)
    zbar = np.empty(rows, np.int32)
    umin = np.empty(rows, np.float32) if u_range is None else _c(u_range[0], np.float32).copy()
    umax = np.empty(rows, np.float32) if u_range is None else _c(u_range[1], np.float32).copy()
    sat = lib().ora_merge_mul(rows, n, r, u_bits, _p(wround), _p(z), _p(s), _p(rstar), _p(A), _p(B), _p(m), _p(ur),
                              _p(sbar), _p(zbar), _p(umin), _p(umax), 0 if u_range is None else 1)
    return dict(m=m, uround=ur, sbar=sbar, zbar=zbar, umin=umin, umax=umax, sat=int(sat))


def log2_round(a: float) -> int:
    return int(lib().ora_log2_round(float(a)))


def log2_round_batch(a):
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.int32)
    lib().ora_log2_round_batch(a.size, _p(a), _p(out))
    return out


def merge_shift(wround, z, s, rstar, A, B, w_bits, v_bits, u_range=None):
    """u_range: optional (u_min, u_max) per row, used in place of the row's own range."""
    wround = _c(wround, np.uint8)
    rows, n = wround.shape
    A = _c(A, np.float32)
    B = _c(B, np.float32)
    r = A.shape[1]
    assert A.shape == (rows, r) and B.shape == (r, n)
    z, s, rstar = _c(z, np.int32), _c(s, np.float32), _c(rstar, np.float32)
    m = np.empty((rows, n), np.int8)
    sh = np.empty((rows, n), np.uint8)
    sbar = np.empty(rows, np.float32)
    umin = np.empty(rows, np.float32) if u_range is None else _c(u_range[0], np.float32).copy()
    umax = np.empty(rows, np.float32) if u_range is None else _c(u_range[1], np.float32).copy()
    sat = lib().ora_merge_shift(rows, n, r, w_bits, v_bits, _p(wround), _p(z), _p(s), _p(rstar), _p(A), _p(B), _p(m),
                                _p(sh), _p(sbar), _p(umin), _p(umax), 0 if u_range is None else 1)
    return dict(m=m, shift=sh, sbar=sbar, umin=umin, umax=umax, sat=int(sat))


def ptq_merge(wround, z, s, rstar, A, B, bits, want_x=False):
    """QLoRA-style comparison path: x = (s*(W_round - z) + R*) + AB in binary32, then
    the base quantizer per row at `bits` (codes, s', z').  The flow IntLoRA removes."""
    wround = _c(wround, np.uint8)
    rows, n = wround.shape
    A = _c(A, np.float32)
    B = _c(B, np.float32)
    r = A.shape[1]
    assert A.shape == (rows, r) and B.shape == (r, n)
    z, s, rstar = _c(z, np.int32), _c(s, np.float32), _c(rstar, np.float32)
    code = np.empty((rows, n), np.uint8)
    sq = np.empty(rows, np.float32)
    zq = np.empty(rows, np.int32)
    x = np.empty((rows, n), np.float32) if want_x else None
    lib().ora_ptq_merge(rows, n, r, bits, _p(wround), _p(z), _p(s), _p(rstar), _p(A), _p(B), _p(code), _p(sq),
                        _p(zq), _p(x))
    return dict(code=code, s=sq, z=zq, x=x)


# --------------------------------------------------------------------------- linear
def quant_act(X):
    X = _c(X, np.float32)
    M, n = X.shape
    xq = np.empty((M, n), np.int8)
    sx = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    lib().ora_quant_act(M, n, _p(X), _p(xq), _p(sx), _p(rs))
    return xq, sx, rs


def bf16_rne(y: float) -> int:
    return int(lib().ora_bf16_rne(float(y)))


def linear(xq, sx, m, sbar, want_exact=True):
    xq = _c(xq, np.int8)
    M, n = xq.shape
    m = _c(m, np.int32)
    d = m.shape[0]
    assert m.shape == (d, n)
    sx, sbar = _c(sx, np.float32), _c(sbar, np.float32)
    exact = np.empty((M, d), np.int64) if want_exact else None
    y32 = np.empty((M, d), np.float32)
    y = np.empty((M, d), np.uint16)
    lib().ora_linear(M, d, n, _p(xq), _p(sx), _p(m), _p(sbar), _p(exact), _p(y32), _p(y))
    return exact, y32, y


def linear_sampled(ts, is_, xq, sx, m, sbar):
    ts = _c(ts, np.int64)
    is_ = _c(is_, np.int64)
    xq = _c(xq, np.int8)
    m = _c(m, np.int32)
    n = xq.shape[1]
    assert m.shape[1] == n
    sx, sbar = _c(sx, np.float32), _c(sbar, np.float32)
    exact = np.empty(ts.size, np.int64)
    y = np.empty(ts.size, np.uint16)
    lib().ora_linear_sampled(ts.size, _p(ts), _p(is_), n, _p(xq), _p(sx), _p(m), _p(sbar), _p(exact), _p(y))
    return exact, y


def byte_planes(m, split=None):
    """Byte split of int16 merged integers into the two int8 GEMM planes, per row.

    Bias split (split 1, and every row when `split` is None): hi = m >> 8,
    lo = (m & 0xFF) - 128, so m = 256*hi + lo + 128 for every int16.
    Balanced split (split 0): hi = (m + 128) >> 8, lo = m - 256*hi, so m = 256*hi + lo;
    both fit int8 only when m <= 32639, which is what a row's split code 0 asserts.
    """
    m = np.asarray(m).astype(np.int32)
    hi = m >> 8
    lo = (m & 0xFF) - 128
    if split is not None:
        bal = np.asarray(split).reshape(-1) == 0
        if m.ndim == 1:
            bal = bal[0] if bal.size == 1 else bal
        else:
            bal = bal[:, None]
        hb = (m + 128) >> 8
        hi = np.where(bal, hb, hi)
        lo = np.where(bal, m - 256 * hb, lo)
    assert hi.min(initial=0) >= -128 and hi.max(initial=0) <= 127, "a balanced row holds m > 32639"
    return hi.astype(np.int8), lo.astype(np.int8)


def plane_split(m):
    """Per-row split code for the int16 GEMM: 0 (balanced) when every m of the row is at
    most 32639, else 1 (bias)."""
    m = np.asarray(m).astype(np.int32)
    return (m >= 32640).any(axis=1).astype(np.uint8)


def plane_store(m, z, zbar, w_bits, u_bits):
    """Byte-plane storage of MUL merged integers (rows x n, n a multiple of 16), as the
    linear layer's int8 matrix cores take them ([IntLoRA notes] "two implementation
    variants", MUL; the int16 values as two int8 byte planes).  Reading of the storage:
    per row, the split is fixed before any element is known, from the bound
    |m| <= max(|z|, |2^w_bits - 1 - z|) * max(z_bar, 2^u_bits - 1 - z_bar):
      bound <= 32639: balanced split (hi = (m + 128) >> 8, lo = m - 256 hi);
      otherwise:      bias split (hi = m >> 8, lo = (m & 0xFF) - 128).
    Layout: per row, the n high bytes (column order), then the n low bytes.  Code: 3
    for a bias row; for a balanced row 1 if some high byte is not zero, else 0.
    Returns (layout uint8 rows x 2n, codes uint8)."""
    m = np.asarray(m).astype(np.int64)
    rows, n = m.shape
    assert n % 16 == 0
    z = np.asarray(z, np.int64).reshape(-1)
    zbar = np.asarray(zbar, np.int64).reshape(-1)
    wmax, umax = (1 << w_bits) - 1, (1 << u_bits) - 1
    bound = np.maximum(np.abs(z), np.abs(wmax - z)) * np.maximum(zbar, umax - zbar)
    bias = bound > 32639
    hi, lo = byte_planes(m, split=bias.astype(np.uint8))
    code = np.where(bias, 3, np.where((hi != 0).any(axis=1), 1, 0)).astype(np.uint8)
    layout = np.concatenate([hi, lo], axis=1).astype(np.int8)
    return np.ascontiguousarray(layout).view(np.uint8), code


def merged_from_planes(layout, code):
    """The merged integers a byte-plane layout stores: 256 hi + lo (+ 128 on bias rows)."""
    layout = np.ascontiguousarray(layout, np.uint8)
    n = layout.shape[1] // 2
    planes = layout.view(np.int8).astype(np.int64)
    hi, lo = planes[:, :n], planes[:, n:]
    bias = ((np.asarray(code, np.uint8) >> 1) & 1).astype(np.int64)[:, None]
    return 256 * hi + lo + 128 * bias


def merged_from_codes(ucode, wround, z, zbar):
    """The merged integers re-formed from stored codes ([IntLoRA notes] "两种实现版本",
    MUL: W' = s_bar (U_round - z_bar) (.) (W_round - z)): m = (U_round - z_bar) *
    (W_round - z) per element, saturated to int16 as the merge stores it.  The codes
    are unpacked (one code per element); z, zbar are per row."""
    u = np.asarray(ucode).astype(np.int64) - np.asarray(zbar).astype(np.int64)[:, None]
    w = np.asarray(wround).astype(np.int64) - np.asarray(z).astype(np.int64)[:, None]
    return np.clip(u * w, -32768, 32767).astype(np.int16)


def linear_from_codes(xq, sx, ucode, wround, z, zbar, sbar, want_exact=True):
    """Merge-on-load linear layer: the integer linear layer (``linear``) on the merged
    integers formed from U's codes and the base codes (``merged_from_codes``)."""
    return linear(xq, sx, merged_from_codes(ucode, wround, z, zbar), sbar, want_exact)
