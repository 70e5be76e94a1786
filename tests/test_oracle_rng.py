"""Pins of the oracle's random-number side (CPU only).

- Philox4x32-10 against an independent implementation: rocRAND's engine, compiled from
  its public header (tests/helpers/rocrand_philox_ref.cpp).
- Counter mapping: R depends only on (seed, layer_id, i, j) -- row blocks regenerate
  the same values ([IntLoRA notes] section "1. AQS": R is regenerated from a fixed
  seed, so it needs no storage).
- Laplace sampling ([IntLoRA summary]: Laplace is the retained distribution for R):
  moments, a Kolmogorov-Smirnov test and exact symmetry of the inverse CDF.
- The binary32 log is correctly rounded on its whole input domain (the 2^22 odd
  multiples of 2^-23 in (0, 1)), checked against 40-digit decimal logarithms where the
  binary64 value is near a rounding midpoint.
"""
import decimal
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))


def _philox_ref_binary():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    out = os.path.join(tempfile.gettempdir(), "intlora_philox_ref_%d" % os.getpid())
    if not os.path.exists(out):
        subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950",
                        os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp"), "-o", out],
                       check=True, capture_output=True, cwd=tempfile.gettempdir())
    return out


def test_philox_matches_rocrand_engine(ora):
    rng = np.random.Generator(np.random.PCG64(12345))
    N = 4096
    rec = rng.integers(0, 2**32, size=(N, 6), dtype=np.uint64).astype(np.uint32)
    # include the structured corners: zero and all-ones counters / keys
    rec[0] = 0
    rec[1] = 0xFFFFFFFF
    rec[2, :4] = [1, 0, 0, 0]
    rec[2, 4:] = 0
    ref_bin = _philox_ref_binary()
    with tempfile.TemporaryDirectory() as td:
        fin, fout = os.path.join(td, "in.bin"), os.path.join(td, "out.bin")
        rec.tofile(fin)
        subprocess.run([ref_bin, fin, fout], check=True)
        ref = np.fromfile(fout, dtype=np.uint32).reshape(N, 4)
    got = ora.philox(rec[:, :4], rec[:, 4:])
    assert np.array_equal(got, ref)


def test_r_rows_regenerate_identically(ora):
    d, n = 37, 53
    c = np.linspace(0.5, 2.0, d).astype(np.float32)
    full = ora.gen_r(d, n, 7, 3, c)
    for row0, rows in [(0, 1), (5, 9), (36, 1), (11, 26)]:
        part = ora.gen_r_rows(row0, rows, n, 7, 3, c[row0:row0 + rows])
        assert np.array_equal(part.view(np.uint32), full[row0:row0 + rows].view(np.uint32))
    # seed and layer id both select a different stream
    assert not np.array_equal(full, ora.gen_r(d, n, 8, 3, c))
    assert not np.array_equal(full, ora.gen_r(d, n, 7, 4, c))


def test_counter_layout_word_selection(ora):
    """Element q uses word q & 3 of the block with counter (q >> 2, q >> 34, layer, 0)."""
    d, n = 3, 10
    seed, layer = 0x1234_5678_9ABC_DEF0, 5
    c = np.ones(d, np.float32)
    R = ora.gen_r(d, n, seed, layer, c).ravel()
    for q in range(d * n):
        ctr = np.array([[q >> 2, 0, layer, 0]], np.uint32)
        key = np.array([[seed & 0xFFFFFFFF, seed >> 32]], np.uint32)
        word = ora.philox(ctr, key)[0, q & 3]
        assert R[q] == ora.laplace(np.array([word], np.uint32))[0]


def test_uniform_words_chi2(ora):
    d, n = 64, 4096
    words = []
    key = np.array([[0, 0]], np.uint32)
    ctr = np.zeros((d * n // 4, 4), np.uint32)
    ctr[:, 0] = np.arange(d * n // 4, dtype=np.uint32)
    out = ora.philox(ctr, np.repeat(key, ctr.shape[0], axis=0)).ravel()
    top = (out >> 24).astype(np.int64)  # 256 bins
    counts = np.bincount(top, minlength=256)
    chi2, p = stats.chisquare(counts)
    assert p > 1e-4, (chi2, p)
    words.append(out)


def test_laplace_moments_and_ks(ora):
    c = np.ones(256, np.float32)
    L = ora.gen_r(256, 4096, 0, 0, c).ravel().astype(np.float64)
    N = L.size
    # Laplace(0, 1): mean 0, variance 2, excess kurtosis 3
    assert abs(L.mean()) < 5 * np.sqrt(2.0 / N)
    var_sd = np.sqrt((24.0 - 4.0) / N)  # var of sample variance ~ (mu4 - sigma^4)/N, mu4 = 24
    assert abs(L.var() - 2.0) < 5 * var_sd
    ks = stats.kstest(L[:200000], stats.laplace(loc=0.0, scale=1.0).cdf)
    assert ks.pvalue > 1e-4, ks


def test_laplace_inverse_cdf_is_antisymmetric(ora):
    """Words a and 2^23 - 1 - a (top 23 bits) give u and 1 - u, so L flips sign exactly."""
    rng = np.random.Generator(np.random.PCG64(3))
    a = rng.integers(0, 2**23, size=100000, dtype=np.uint64).astype(np.uint32)
    low = rng.integers(0, 2**9, size=a.size, dtype=np.uint64).astype(np.uint32)
    w1 = (a << 9) | low
    w2 = ((np.uint32(2**23 - 1) - a) << 9) | low
    L1 = ora.laplace(w1)
    L2 = ora.laplace(w2)
    assert np.array_equal(L1, -L2)
    # extreme words: the smallest g is 2^-23, so |L| <= 23 ln 2
    ext = ora.laplace(np.array([0, 0xFFFFFFFF, 0x7FFFFFFF, 0x80000000], np.uint32))
    assert np.all(np.abs(ext) <= np.float32(23 * np.log(2.0)) * (1 + 1e-6))
    assert ext[0] == -ext[1]


def _rn32_of_decimal(x: decimal.Decimal) -> np.float32:
    """Round a decimal to the nearest binary32, ties to even (exact)."""
    import fractions
    f = fractions.Fraction(x)
    lo = np.float32(float(f))
    # adjust lo to the binary32 at or below f
    while fractions.Fraction(float(lo)) > f:
        lo = np.nextafter(lo, np.float32(-np.inf))
    while fractions.Fraction(float(np.nextafter(lo, np.float32(np.inf)))) <= f:
        lo = np.nextafter(lo, np.float32(np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    dl = f - fractions.Fraction(float(lo))
    dh = fractions.Fraction(float(hi)) - f
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (lo.view(np.uint32) & 1) == 0 else hi


def test_ln_correctly_rounded_on_whole_domain(ora):
    # every g the Laplace sampler can produce: odd multiples of 2^-23 in (0, 1)
    g = (np.arange(1, 2**23, 2, dtype=np.float64) * 2.0**-23).astype(np.float32)
    got = ora.ln_rn32(g)
    l64 = np.log(g.astype(np.float64))
    r32 = l64.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), r32.view(np.uint32))
    # where the binary64 value lies close to a binary32 midpoint, decide with 40 digits
    up = np.nextafter(r32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r32, np.float32(-np.inf)).astype(np.float64)
    r64 = r32.astype(np.float64)
    mid_lo = (r64 + dn) / 2.0
    mid_hi = (r64 + up) / 2.0
    margin = np.minimum(np.abs(l64 - mid_lo), np.abs(l64 - mid_hi)) / np.abs(l64)
    close = np.nonzero(margin < 2.0**-45)[0]
    decimal.getcontext().prec = 40
    for idx in close:
        exact = decimal.Decimal(float(g[idx])).ln()
        assert _rn32_of_decimal(exact) == got[idx], (g[idx], got[idx])
    # and a random sample of ordinary points against the 40-digit log
    rng = np.random.Generator(np.random.PCG64(9))
    for idx in rng.integers(0, g.size, 200):
        exact = decimal.Decimal(float(g[idx])).ln()
        assert _rn32_of_decimal(exact) == got[idx]
