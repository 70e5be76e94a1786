"""Seeded synthetic inputs for the IntLoRA merge and integer linear layer.

This module holds no arithmetic of the method: it only draws the raw inputs (the
pretrained fp32 weight W, the LoRA factors A and B, the fp32 activations X) and
describes the layer shapes of the five workloads.  Both the GPU path and the CPU
oracle are fed from it.  The auxiliary matrix R is not drawn here: each side
regenerates it from (seed, layer_id) with its own Philox4x32-10.

Workloads (shapes are out x in = d x n; the pages measure on SD v1.5, FLUX.1 and
Llama-3-8B, none of which is available; these synthetic tensors take their layer
shapes):
  0  single 320x320 linear, W8A8, MUL U 8-bit, r = 4, M = 64
  1  SD v1.5 UNet 640-channel attention + GEGLU FF layers, W4A8, r = 4,
     MUL (U 4-bit) and SHIFT (log2 4-bit), M = 2 x 1024
  2  SD v1.5 UNet 320-channel layers incl. cross-attention k/v, W8A8, r = 4,
     SHIFT (log2 4-bit), M = 2 x 4096
  3  FLUX-like DiT block linears (hidden 3072), W4A8, MUL U 4-bit, r = 32,
     M = 4608, W with 0.1% heavy-tail entries x8
  4  Llama-3-8B projection shapes, W8A8, MUL U 8-bit, r = 64, M = 2048 and 16,
     plus a merge-only sweep over 32 layers x 7 matrices

Distributions: W ~ N(0, sigma^2) (sigma = 0.02, 0.015 for workload 3),
A ~ N(0, 1/4), B ~ N(0, 1e-3) (second argument = variance, as in the W notation),
X ~ N(0, 1) with two seeded outlier columns scaled x10.  Philox seed 0, layer_id =
layer index (7 * layer + matrix in the Llama sweep), VMC alpha = 1.5.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ALPHA = 1.5
PHILOX_SEED = 0


@dataclass(frozen=True)
class Layer:
    name: str
    d: int  # out_features
    n: int  # in_features


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    layers: tuple
    w_bits: int
    modes: tuple  # (("mul", u_bits) | ("shift", v_bits), ...)
    r: int
    tokens: tuple  # M values
    w_std: float = 0.02
    tail_p: float = 0.0
    tail_scale: float = 1.0
    sweep_layers: int = 0
    extra: dict = field(default_factory=dict)


def _L(name, d, n):
    return Layer(name, d, n)


WORKLOADS = {
    0: Workload(0, "single_linear_320x320_w8a8_mul_r4", (_L("linear", 320, 320),), 8, (("mul", 8),), 4, (64,)),
    1: Workload(1, "sd15_unet_640ch_w4a8_mul_shift_r4",
                (_L("q", 640, 640), _L("k", 640, 640), _L("v", 640, 640), _L("o", 640, 640),
                 _L("ff_geglu_in", 5120, 640), _L("ff_out", 640, 2560)),
                4, (("mul", 4), ("shift", 4)), 4, (2048,)),
    2: Workload(2, "sd15_unet_320ch_w8a8_shift_r4",
                (_L("q", 320, 320), _L("k", 320, 320), _L("v", 320, 320), _L("o", 320, 320),
                 _L("xattn_k", 320, 768), _L("xattn_v", 320, 768), _L("ff_geglu_in", 2560, 320),
                 _L("ff_out", 320, 1280)),
                8, (("shift", 4),), 4, (8192,)),
    3: Workload(3, "flux_dit_block_w4a8_mul_r32",
                (_L("qkv", 9216, 3072), _L("out", 3072, 3072), _L("mlp_in", 12288, 3072), _L("mlp_out", 3072, 12288)),
                4, (("mul", 4),), 32, (4608,), w_std=0.015, tail_p=0.001, tail_scale=8.0),
    4: Workload(4, "llama3_8b_w8a8_mul_r64",
                (_L("q", 4096, 4096), _L("k", 1024, 4096), _L("v", 1024, 4096), _L("o", 4096, 4096),
                 _L("gate", 14336, 4096), _L("up", 14336, 4096), _L("down", 4096, 14336)),
                8, (("mul", 8),), 64, (2048, 16), sweep_layers=32),
}


def layer_seed(workload: int, layer_index: int) -> int:
    return 1000 * workload + layer_index


def layer_id(workload: int, layer_index: int, block: int = 0) -> int:
    """Philox layer id: the layer index; in the Llama sweep 7 * block + matrix."""
    if workload == 4:
        return 7 * block + layer_index
    return layer_index


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def weight(wl: Workload, layer_index: int, d: int | None = None, n: int | None = None, block: int = 0) -> np.ndarray:
    """Pretrained fp32 weight W (d x n) of one layer."""
    L = wl.layers[layer_index]
    d = L.d if d is None else d
    n = L.n if n is None else n
    rng = _rng(layer_seed(wl.index, layer_index) + 100000 * block)
    W = rng.standard_normal((d, n), dtype=np.float32) * np.float32(wl.w_std)
    if wl.tail_p > 0.0:
        mask = rng.random((d, n), dtype=np.float32) < np.float32(wl.tail_p)
        W[mask] *= np.float32(wl.tail_scale)
    return W


SWEEP_CHUNK = 256  # rows per independently seeded chunk of a sweep weight


def sweep_weight(wl: Workload, layer_index: int, block: int, rows=None, threads: int = 16) -> np.ndarray:
    """Pretrained fp32 weight of matrix `layer_index` of transformer block `block` in the
    merge-only sweep (same law as weight()).  Rows are drawn in chunks of SWEEP_CHUNK,
    each from its own seed, so that chunks are drawn in parallel threads and a sample of
    rows is drawn without the rest.  rows: None for the whole d x n matrix, else the
    sorted row indices wanted (returned in that order)."""
    L = wl.layers[layer_index]
    chunks = range((L.d + SWEEP_CHUNK - 1) // SWEEP_CHUNK) if rows is None else \
        sorted({int(i) // SWEEP_CHUNK for i in rows})

    def draw(ch):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((wl.index, layer_index, block, ch, 7))))
        h = min(SWEEP_CHUNK, L.d - ch * SWEEP_CHUNK)
        Wc = rng.standard_normal((h, L.n), dtype=np.float32) * np.float32(wl.w_std)
        if wl.tail_p > 0.0:
            mask = rng.random((h, L.n), dtype=np.float32) < np.float32(wl.tail_p)
            Wc[mask] *= np.float32(wl.tail_scale)
        return Wc

    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max(1, threads)) as ex:
        parts = dict(zip(chunks, ex.map(draw, chunks)))
    if rows is None:
        return np.concatenate([parts[ch] for ch in chunks])
    return np.stack([parts[int(i) // SWEEP_CHUNK][int(i) % SWEEP_CHUNK] for i in rows])


def lora(wl: Workload, layer_index: int, d: int | None = None, n: int | None = None, r: int | None = None,
         block: int = 0):
    """LoRA factors A (d x r) ~ N(0, 1/4) and B (r x n) ~ N(0, 1e-3), fp32."""
    L = wl.layers[layer_index]
    d = L.d if d is None else d
    n = L.n if n is None else n
    r = wl.r if r is None else r
    rng = _rng(layer_seed(wl.index, layer_index) + 500000 + 100000 * block)
    A = rng.standard_normal((d, r), dtype=np.float32) * np.float32(0.5)
    B = rng.standard_normal((r, n), dtype=np.float32) * np.float32(np.sqrt(1e-3))
    return A, B


def activations(wl: Workload, n: int, M: int, layer_index: int = 0) -> np.ndarray:
    """fp32 activations X (M x n) ~ N(0, 1) with 2 seeded outlier columns x10."""
    rng = _rng(layer_seed(wl.index, layer_index) + 900000 + M)
    X = rng.standard_normal((M, n), dtype=np.float32)
    cols = rng.choice(n, size=min(2, n), replace=False)
    X[:, cols] *= np.float32(10.0)
    return X


def random_matrix(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """Generic seeded N(0, std^2) fp32 matrix for small edge-case tests."""
    return _rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)


def random_codes(seed: int, shape, bits: int) -> np.ndarray:
    """Uniform random b-bit unsigned codes (uint8)."""
    return _rng(seed).integers(0, 1 << bits, size=shape, dtype=np.uint8)


def random_ints(seed: int, shape, lo: int, hi: int, dtype=np.int32) -> np.ndarray:
    """Uniform random integers in [lo, hi]."""
    return _rng(seed).integers(lo, hi + 1, size=shape).astype(dtype)


def random_positive(seed: int, shape, lo: float, hi: float) -> np.ndarray:
    """Log-uniform positive fp32 values in [lo, hi]."""
    u = _rng(seed).random(shape)
    return np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.float32)
