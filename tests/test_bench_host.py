"""Host-side helpers of bench.py (CPU): the decoding of the byte-plane storage that the
benchmark's consistency checks and error figures use must agree with the oracle's
storage rule, and the launch-rule mirror must match its own definition on a few shapes."""
import numpy as np
import torch

import bench
import oracle


def test_merged_m_decodes_the_plane_storage():
    rng = np.random.Generator(np.random.PCG64(41))
    d, n = 37, 96
    m = rng.integers(-32768, 32768, size=(d, n))
    z = np.where(np.arange(d) % 2 == 0, 0, 128)  # bias rows (z = 0) beside balanced rows
    m[z == 128] = np.clip(m[z == 128], -16384, 16384)
    m[5] = rng.integers(-100, 101, size=n)  # a balanced row with a zero high plane
    z[5] = 128
    lay, code = oracle.plane_store(m, z, np.full(d, 128), 8, 8)
    assert set(code.tolist()) == {0, 1, 3}
    out = {"planes": torch.from_numpy(lay.copy()), "code": torch.from_numpy(code.copy())}
    got = bench.merged_m({"out": out}, torch)
    assert np.array_equal(got.numpy(), m)


def test_gemm_alg_bytes():
    # activations, stored weights (one byte per multiplied plane, or the SHIFT codes), bf16 outputs
    assert bench.gemm_alg_bytes(16, 4096, 4096, "mul", 8, 2) == 16 * 4096 + 4096 * 4096 * 2 + 2 * 16 * 4096
    assert bench.gemm_alg_bytes(16, 4096, 4096, "mul", 4, 1) == 16 * 4096 + 4096 * 4096 + 2 * 16 * 4096
    assert bench.gemm_alg_bytes(8, 320, 640, "shift", 4, None) == 8 * 640 + 320 * 640 * 0.5 + 2 * 8 * 320
