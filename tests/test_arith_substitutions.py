"""The arithmetic substitutions the GPU kernels rest on, proved on the CPU (no GPU).

[IntLoRA notes] "2. MLA" divides R* + AB by the signed pretrained integer
w = W_round - z, and "two implementation variants" (MUL) quantizes U / s_bar; the
definition of both is the IEEE binary32 division.  The kernels replace each division
by cheaper steps that give the same bits; these tests check that claim against the
division itself, in plain C (tests/helpers/arith_checks.c), exhaustively where the
domain allows it:

1. t / w for 1 <= |w| <= 255 as q0 = RN(t y), r = fma(-q0, w, t), q = fma(r, y, q0)
   with y = RN(1/w), for every binary32 significand of t, both signs, at the bottom
   and top of the window 2^-100 <= |t| <= 2^100 and at exponents in between.  The
   steps scale exactly with t's exponent inside the window: q0 stays normal
   (|q0| >= 2^-108), the residual r is an exact multiple of ulp(q0) >= 2^-131 (exact
   even where subnormal), and q is one rounding of an exact value; so the exponents
   checked cover the window.
2. The MUL code from qt = RN(u RN(1/s)) instead of RN(u / s), whenever |qt| < 512 and
   qt is more than 2^-11 from every half-integer, at every half-integer boundary of
   the code range (u within 40 ulps of each boundary) for scales across the binary32
   exponent range, and on random u in the range of 2- to 8-bit codes.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def helper():
    global _lib
    if _lib is None:
        out = os.path.join(tempfile.gettempdir(), "intlora_arith_checks_%d.so" % os.getpid())
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-march=native", "-fopenmp", "-fPIC",
                        "-shared", "-o", out, os.path.join(HERE, "helpers", "arith_checks.c"), "-lm"], check=True)
        L = ctypes.CDLL(out)
        L.count_div_mismatches.restype = ctypes.c_int64
        L.count_div_mismatches.argtypes = [ctypes.c_int] * 4 + [ctypes.c_uint32] * 2 + [ctypes.POINTER(ctypes.c_int64)]
        L.count_div_mismatches_pow2.restype = ctypes.c_int64
        L.count_div_mismatches_pow2.argtypes = [ctypes.c_int]
        L.count_code_mismatches.restype = ctypes.c_int64
        L.count_code_mismatches.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        L.count_code_mismatches_random.restype = ctypes.c_int64
        L.count_code_mismatches_random.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                                   ctypes.POINTER(ctypes.c_int64)]
        L.fmaf_chain.restype = None
        L.fmaf_chain.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int] + [ctypes.c_void_p] * 3
        _lib = L
    return _lib


# t = 2^e m: biased exponent 127 + e.  The window's ends (e = -100 and e = 99, whose
# binade reaches 2^100) and exponents in between, each over every significand.
@pytest.mark.parametrize("e", [-100, -99, -37, -1, 0, 1, 42, 98, 99])
def test_div_small_int_equals_ieee_division(e):
    L = helper()
    n = ctypes.c_int64()
    bad = L.count_div_mismatches(-255, 255, 127 + e, 127 + e, 1, 0, ctypes.byref(n))
    assert n.value == 510 * (1 << 23) * 2
    assert bad == 0


def test_div_small_int_window_edges_powers_of_two():
    L = helper()
    for e in (-100, 100):
        assert L.count_div_mismatches_pow2(e) == 0


def test_div_small_int_fails_outside_the_window():
    """The window is not vacuous: far below it (subnormal quotients) the steps differ
    from the division for some t, which is why the kernels take the IEEE division
    there."""
    L = helper()
    n = ctypes.c_int64()
    assert L.count_div_mismatches(3, 255, 1, 1, 4093, 7, ctypes.byref(n)) > 0  # a sample (subnormals are slow)


def _scales():
    rng = np.random.Generator(np.random.PCG64(2024))
    mant = rng.integers(0, 1 << 23, size=3000, dtype=np.uint32)
    expo = rng.integers(1, 254, size=3000, dtype=np.uint32)
    s = ((expo << 23) | mant).view(np.float32)
    extra = np.array([1.0, 1.5, 2.0 / 3.0, 1.0 / 255.0, 2.0 ** -126, 2.0 ** -100, 2.0 ** 100,
                      float.fromhex('0x1.fffffep127'), 3.0e-5], np.float32)
    return np.ascontiguousarray(np.concatenate([s, extra]).astype(np.float32))


def test_mul_code_fast_rule_at_every_half_integer():
    L = helper()
    s = _scales()
    fast, total = ctypes.c_int64(), ctypes.c_int64()
    bad = L.count_code_mismatches(s.size, s.ctypes.data, 40, ctypes.byref(fast), ctypes.byref(total))
    assert bad == 0
    assert total.value > 10 ** 7
    # near the boundaries the rule defers to the division often, but not always
    assert 0.05 * total.value < fast.value < total.value


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_mul_code_fast_rule_random(bits):
    L = helper()
    s = _scales()
    fast = ctypes.c_int64()
    per = 4000
    bad = L.count_code_mismatches_random(s.size, s.ctypes.data, bits, per, ctypes.byref(fast))
    assert bad == 0
    assert fast.value > 0.9 * s.size * per * 0.9  # the fast rule decides almost every code
