"""Pins of the merge-on-load linear layer's oracle (CPU): forming the merged integers
from U's stored codes and the base codes reproduces, bit for bit, the merged integers
and the linear layer of the materialized MUL merge (whose m is formed in the C oracle)."""
import numpy as np
import pytest

import oracle


def _state(seed, d, n, r, w_bits):
    g = np.random.Generator(np.random.PCG64(seed))
    W = g.normal(0.0, 0.02, (d, n)).astype(np.float32)
    st = oracle.setup_layer(W, seed, 3, w_bits)
    A = g.normal(0.0, 0.5, (d, r)).astype(np.float32)
    Bm = g.normal(0.0, 0.03, (r, n)).astype(np.float32)
    return st, A, Bm


@pytest.mark.parametrize("d,n,r,w_bits,u_bits", [(24, 64, 4, 4, 4), (40, 96, 8, 4, 3), (16, 64, 4, 8, 4),
                                                 (33, 128, 16, 8, 8), (8, 32, 2, 4, 2)])
def test_codes_reproduce_materialized_merge(d, n, r, w_bits, u_bits):
    st, A, Bm = _state(100 + d + n, d, n, r, w_bits)
    mm = oracle.merge_mul(st["wround"], st["z"], st["s"], st["rstar"], A, Bm, u_bits)
    m2 = oracle.merged_from_codes(mm["uround"], st["wround"], st["z"], mm["zbar"])
    assert np.array_equal(m2, mm["m"])
    w = st["wround"].astype(np.int64) - st["z"].astype(np.int64)[:, None]
    assert np.all(mm["uround"][w == 0] == np.broadcast_to(mm["zbar"][:, None], w.shape)[w == 0])
    g = np.random.Generator(np.random.PCG64(d))
    X = g.normal(0.0, 1.0, (19, n)).astype(np.float32)
    xq, sx, _ = oracle.quant_act(X)
    e1, y1_32, y1 = oracle.linear(xq, sx, mm["m"], mm["sbar"])
    e2, y2_32, y2 = oracle.linear_from_codes(xq, sx, mm["uround"], st["wround"], st["z"], mm["zbar"], mm["sbar"])
    assert np.array_equal(e1, e2) and np.array_equal(y1, y2)


def test_four_bit_codes_bound_the_merged_integers():
    """With 4-bit U and 4-bit base codes |m| <= 15 * 15, so no element saturates and
    every row takes the balanced byte split."""
    u = np.arange(16, dtype=np.uint8)
    U, Wc = np.meshgrid(u, u)
    for zb in range(16):
        for zw in range(16):
            m = oracle.merged_from_codes(U.reshape(1, -1), Wc.reshape(1, -1), np.array([zw]), np.array([zb]))
            assert np.abs(m.astype(np.int32)).max() <= 225
            assert oracle.plane_split(m)[0] == 0


def test_saturation_matches_the_merge():
    """8-bit codes can overflow int16: the re-formed value saturates exactly as the
    merge's stored m (both clamp the exact product)."""
    ucode = np.array([[255, 0, 255, 0]], np.uint8)
    wc = np.array([[255, 255, 0, 0]], np.uint8)
    m = oracle.merged_from_codes(ucode, wc, np.array([0]), np.array([0]))
    assert m.tolist() == [[32767, 0, 0, 0]]
    m = oracle.merged_from_codes(ucode, wc, np.array([255]), np.array([0]))
    assert m.tolist() == [[0, 0, -32768, 0]]
