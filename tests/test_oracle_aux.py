"""Pins of the oracle's other auxiliary-matrix laws (CPU only): the Gaussian, Cauchy and
Student-t(2) samplers of the distribution ablation ([IntLoRA summary], table "Measured
effects": Laplace against Gaussian, Cauchy and Student-t auxiliary matrices).

- Each law against its closed form: scipy's inverse distribution functions of the Cauchy
  and Student-t(2) laws at the sampler's uniform, and the Box-Muller identities
  S^2 = -2 ln u1, atan2(sine sample, cosine sample) = 2 pi u2 for the Gaussian pairs.
- Every transcendental step is correctly rounded to binary32 on its whole input domain
  (the 2^23 arguments the sampler can produce): where the oracle's binary64 value lies
  near a binary32 midpoint, a 40-digit evaluation decides.
- Distribution sanity on a large sample: moments and Kolmogorov-Smirnov tests.
- VMC for the other laws (reading: sigma_R = 1) in closed form, and R* = c * sample.
"""
import numpy as np
import pytest
from scipy import stats

import oracle

mpmath = pytest.importorskip("mpmath")

U_INDEX = np.arange(2**23, dtype=np.uint64)  # a = floor(x / 2^9)


def _uniform(a):
    return (2.0 * a.astype(np.float64) + 1.0) * 2.0**-24


def _rn32_exact(x):
    """Nearest binary32 (ties to even) of an mpmath number."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(mpmath.mpf(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def _midpoint_margin(v64):
    r32 = v64.astype(np.float32)
    up = np.nextafter(r32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r32, np.float32(-np.inf)).astype(np.float64)
    r64 = r32.astype(np.float64)
    m = np.minimum(np.abs(v64 - (r64 + dn) / 2.0), np.abs(v64 - (r64 + up) / 2.0))
    return m / np.maximum(np.abs(v64), 1e-300)


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_trig_correctly_rounded_on_whole_domain(kind):
    # cos / sin take v = 2 u2 = (2a + 1) 2^-23 in (0, 2); tan takes v = u - 1/2 = N 2^-24
    a = U_INDEX
    if kind < 2:
        v = (2.0 * a.astype(np.float64) + 1.0) * 2.0**-23
    else:
        v = (2.0 * a.astype(np.float64) + 1.0 - 2.0**23) * 2.0**-24
    got = oracle.trig_pi(v, kind)
    # against numpy's binary64 functions of the same exactly reduced points: agreement
    # to a few units of 2^-52 everywhere except near the zeros, which the reduction
    # resolves and the exact check below covers
    ref = np.cos(np.pi * v) if kind == 0 else np.sin(np.pi * v) if kind == 1 else np.tan(np.pi * v)
    # numpy's error is the argument's rounding (pi v) times the derivative
    ok = (np.abs(ref) > 1e-3) & (np.abs(ref) < 1e3)
    deriv = np.abs(np.sin(np.pi * v)) if kind == 0 else np.abs(np.cos(np.pi * v)) if kind == 1 else 1.0 + ref * ref
    tol = 1e-15 * np.abs(ref) + 4.0 * 2.0**-53 * np.pi * np.abs(v) * deriv
    assert np.all(np.abs(got[ok] - ref[ok]) <= tol[ok])
    # the binary32 rounding equals RN32 of the exact value: exact check where close to a
    # midpoint, and on a random sample of ordinary points and of points near the zeros
    mpmath.mp.dps = 40
    fn = [mpmath.cospi, mpmath.sinpi, lambda x: mpmath.tan(mpmath.pi * x)][kind]
    margin = _midpoint_margin(got)
    close = np.nonzero(margin < 2.0**-44)[0]
    rng = np.random.Generator(np.random.PCG64(17 + kind))
    extra = np.concatenate([rng.integers(0, v.size, 300), np.nonzero(~ok)[0][:200]])
    for idx in np.concatenate([close, extra]):
        exact = fn(mpmath.mpf(float(v[idx])))
        assert _rn32_exact(exact) == np.float32(got[idx]), (kind, v[idx], got[idx])


def test_gaussian_log_correctly_rounded_at_bias_24():
    # the Gaussian's ln u1 with u1 = (2a + 1) 2^-24: the binary64 log rounded once
    u1 = _uniform(U_INDEX)
    l64 = np.log(u1)
    margin = _midpoint_margin(l64)
    close = np.nonzero(margin < 2.0**-44)[0]
    mpmath.mp.dps = 40
    for idx in close:
        assert _rn32_exact(mpmath.log(mpmath.mpf(float(u1[idx])))) == np.float32(l64[idx])
    # and the oracle's sampler uses exactly that value: S^2 = -2 L up to S's rounding
    w = np.zeros((64, 4), np.uint32)
    w[:, 0] = (np.arange(64, dtype=np.uint32) * 131071) << 9
    w[:, 1] = 0
    out = oracle.aux_samples(w, 1)
    S = np.float32(np.sqrt(np.float32(-2.0) * np.log(_uniform(w[:, 0].astype(np.uint64) >> 9)).astype(np.float32)))
    # cos(2 pi u2) at u2 = 2^-24 is 1 - 2e-13: C rounds to 1, so sample = S exactly
    assert np.array_equal(out[:, 0], S)


def _words_for(a_values, rng):
    low = rng.integers(0, 512, a_values.size, dtype=np.uint32)
    return (a_values.astype(np.uint32) << np.uint32(9)) | low


def test_cauchy_and_student_t2_are_their_inverse_cdfs():
    rng = np.random.Generator(np.random.PCG64(3))
    a = np.concatenate([np.arange(0, 4096), rng.integers(0, 2**23, 200000), np.arange(2**23 - 4096, 2**23)])
    u = _uniform(a.astype(np.uint64))
    w = np.zeros((a.size, 4), np.uint32)
    w[:, 0] = _words_for(a, rng)
    cau = oracle.aux_samples(w, 2)[:, 0].astype(np.float64)
    t2 = oracle.aux_samples(w, 3)[:, 0].astype(np.float64)
    ref_c = stats.cauchy.ppf(u)
    ref_t = stats.t(2).ppf(u)
    assert np.all(np.abs(cau - ref_c) <= 2.0**-22 * np.abs(ref_c) + 1e-30)
    assert np.all(np.abs(t2 - ref_t) <= 2.0**-22 * np.abs(ref_t) + 1e-30)
    # odd symmetry: u -> 1 - u negates the sample exactly
    w2 = w.copy()
    w2[:, 0] = _words_for((2**23 - 1 - a).astype(np.uint32), rng)
    assert np.array_equal(oracle.aux_samples(w2, 2)[:, 0], -oracle.aux_samples(w, 2)[:, 0])
    assert np.array_equal(oracle.aux_samples(w2, 3)[:, 0], -oracle.aux_samples(w, 3)[:, 0])


def test_gaussian_box_muller_identities():
    rng = np.random.Generator(np.random.PCG64(5))
    blocks = rng.integers(0, 2**32, (100000, 4), dtype=np.uint64).astype(np.uint32)
    z = oracle.aux_samples(blocks, 1).astype(np.float64)
    for p in range(2):
        u1 = _uniform(blocks[:, 2 * p].astype(np.uint64) >> 9)
        u2 = _uniform(blocks[:, 2 * p + 1].astype(np.uint64) >> 9)
        c, s = z[:, 2 * p], z[:, 2 * p + 1]
        r2 = c * c + s * s
        assert np.all(np.abs(r2 - (-2.0 * np.log(u1))) <= 2.0**-20 * np.maximum(r2, 1e-6) + 1e-9)
        ang = np.mod(np.arctan2(s, c), 2.0 * np.pi)
        far = r2 > 1e-6
        d = np.abs(ang - 2.0 * np.pi * u2)
        d = np.minimum(d, 2.0 * np.pi - d)
        assert np.all(d[far] <= 1e-5)


@pytest.mark.parametrize("dist,law", [(1, stats.norm), (2, stats.cauchy), (3, stats.t(2))])
def test_laws_by_kolmogorov_smirnov(dist, law):
    rng = np.random.Generator(np.random.PCG64(11))
    blocks = rng.integers(0, 2**32, (50000, 4), dtype=np.uint64).astype(np.uint32)
    x = oracle.aux_samples(blocks, dist).ravel().astype(np.float64)
    assert stats.kstest(x, law.cdf).pvalue > 1e-3
    if dist == 1:
        assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
        # the pair's two samples are uncorrelated
        assert abs(np.corrcoef(x[0::4], x[1::4])[0, 1]) < 0.02


def test_vmc_and_gen_r_for_other_laws():
    sig = np.array([0.5, 1.0, 2.0, 0.015], np.float32)
    for dist in (1, 2, 3):
        assert np.array_equal(oracle.vmc_scale(sig, 0.0, dist), np.ones(4, np.float32))
        assert np.array_equal(oracle.vmc_scale(sig, 1.0, dist), sig)
        c15 = oracle.vmc_scale(sig, 1.5, dist)
        assert np.allclose(c15, sig.astype(np.float64) ** 1.5, rtol=2**-23)
    # Laplace through the law-aware generator is the Laplace generator
    c = np.array([0.3, 1.0, 2.5], np.float32)
    assert np.array_equal(oracle.gen_r_rows(0, 3, 37, 7, 2, c, 0), oracle.gen_r(3, 37, 7, 2, c))
    for dist in (1, 2, 3):
        R = oracle.gen_r(3, 37, 7, 2, c, dist)
        assert np.array_equal(oracle.gen_r_rows(1, 2, 37, 7, 2, c[1:], dist), R[1:])
        # R* = RN32(c * sample): the unit-scale row is the raw sample
        assert np.array_equal(oracle.gen_r(3, 37, 7, 2, np.ones(3, np.float32), dist)[1], R[1])
        assert not np.array_equal(R, oracle.gen_r(3, 37, 7, 2, c, 0))


def test_student_t2_correctly_rounded_on_whole_domain():
    # every u the sampler produces: the binary64 expression rounded once equals RN32 of
    # the exact (2u - 1) / sqrt(2u (1 - u)); 40 digits decide the points near a midpoint
    a = U_INDEX
    w = np.zeros((a.size, 4), np.uint32)
    w[:, 0] = (a.astype(np.uint32) << np.uint32(9))
    got = oracle.aux_samples(w, 3)[:, 0]
    u = _uniform(a)
    v64 = (2.0 * u - 1.0) / np.sqrt(2.0 * u * (1.0 - u))
    assert np.array_equal(got, v64.astype(np.float32))
    close = np.nonzero(_midpoint_margin(v64) < 2.0**-44)[0]
    mpmath.mp.dps = 40
    rng = np.random.Generator(np.random.PCG64(23))
    for idx in np.concatenate([close, rng.integers(0, a.size, 300)]):
        uu = mpmath.mpf(float(u[idx]))
        exact = (2 * uu - 1) / mpmath.sqrt(2 * uu * (1 - uu))
        assert _rn32_exact(exact) == got[idx], (u[idx], got[idx])
