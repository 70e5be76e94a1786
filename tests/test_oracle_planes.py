"""Pins of the oracle's byte-plane storage of the MUL merged integers (CPU).

[IntLoRA notes] "two implementation variants", MUL: the merged integer is
m = (U_round - z_bar)(W_round - z); the int16 values go through the int8 matrix cores
as two byte planes.  The storage fixes each row's split from a bound before any
element is known; these tests check that the bound holds for every code pair, that
the planes reconstruct every int16 exactly under either split, that a code-0 row has
an all-zero high plane, and that the layer's product on the planes equals the
textbook integer product (numpy int64)."""
import itertools

import numpy as np
import pytest

import oracle


def test_bound_covers_every_code_pair():
    """|m| <= max(|z|, |2^bW - 1 - z|) max(z_bar, 2^bU - 1 - z_bar) for every W_round,
    U_round (brute force over 4-bit codes, every zero point pair; 8-bit on a grid)."""
    for wb, ub in ((4, 4), (4, 2), (8, 8)):
        wmax, umax = (1 << wb) - 1, (1 << ub) - 1
        zs = range(wmax + 1) if wb == 4 else range(0, 256, 17)
        zbs = range(umax + 1) if ub <= 4 else range(0, 256, 15)
        for z, zb in itertools.product(zs, zbs):
            w = np.arange(wmax + 1) - z
            u = np.arange(umax + 1) - zb
            mmax = np.abs(np.outer(u, w)).max()
            assert mmax <= max(abs(z), abs(wmax - z)) * max(zb, umax - zb)


def test_planes_reconstruct_every_int16():
    m = np.arange(-32768, 32768, dtype=np.int64).reshape(-1, 16 * 64)  # 64 rows
    z = np.zeros(m.shape[0], np.int32)
    # 8-bit codes with z = 0 and z_bar = 128: bound 255 * 128 > 32639, the bias split
    lay, code = oracle.plane_store(m, z, np.full(m.shape[0], 128), 8, 8)
    assert np.all(code == 3)
    assert np.array_equal(oracle.merged_from_planes(lay, code), m)
    # balanced rows (values up to 32639): 4-bit codes give bound <= 225
    mb = np.clip(m, -32768, 32639)
    lay, code = oracle.plane_store(mb, np.full(m.shape[0], 7), np.full(m.shape[0], 7), 4, 4)
    assert np.all(code == 1)
    assert np.array_equal(oracle.merged_from_planes(lay, code), mb)


def test_code_zero_means_zero_high_plane():
    rng = np.random.Generator(np.random.PCG64(5))
    m = rng.integers(-128, 128, size=(8, 64))
    m[3, 5] = 128  # one row with a value outside int8
    m[6, 7] = -129
    lay, code = oracle.plane_store(m, np.full(8, 7), np.full(8, 8), 4, 4)
    assert list(code) == [0, 0, 0, 1, 0, 0, 1, 0]
    hi = lay.view(np.int8)[:, :64]
    assert np.all(hi[code == 0] == 0)
    assert np.any(hi[3] != 0) and np.any(hi[6] != 0)


def test_layout_whole_row_planes():
    """Row i of the layout: its n high bytes in column order, then its n low bytes; the
    bytes are written out here by hand for one small row (balanced split, 4-bit codes)."""
    m = np.array([[-4000, -129, -128, -1, 0, 1, 127, 128, 255, 256, 300, 1000, 4000, 6000, 7000, 7400]])
    lay, code = oracle.plane_store(m, [7], [7], 4, 4)
    # balanced split: hi = floor((m + 128) / 256), lo = m - 256 hi
    hi = [-16, -1, 0, 0, 0, 0, 0, 1, 1, 1, 1, 4, 16, 23, 27, 29]
    lo = [96, 127, -128, -1, 0, 1, 127, -128, -1, 0, 44, -24, -96, 112, 88, -24]
    assert code[0] == 1
    assert lay.shape == (1, 32)
    assert list(lay[0, :16].view(np.int8)) == hi
    assert list(lay[0, 16:].view(np.int8)) == lo


@pytest.mark.parametrize("bias_rows", [False, True])
def test_linear_on_planes_equals_integer_product(bias_rows):
    rng = np.random.Generator(np.random.PCG64(9))
    d, n, M = 12, 96, 7
    m = rng.integers(-32768, 32640, size=(d, n))
    xq = rng.integers(-127, 128, size=(M, n)).astype(np.int8)
    z = np.where(np.arange(d) % 3 == 0, 0, 100) if bias_rows else np.full(d, 100)
    lay, code = oracle.plane_store(m, z, np.full(d, 128), 8, 8)
    assert (code == 3).any() == bias_rows
    g = lay.view(np.int8).astype(np.int64)
    hi, lo = g[:, :n], g[:, n:]
    x = xq.astype(np.int64)
    exact = 256 * (x @ hi.T) + x @ lo.T + 128 * x.sum(axis=1)[:, None] * ((code >> 1) & 1)[None, :]
    assert np.array_equal(exact, x @ m.T)
