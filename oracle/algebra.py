"""Binary64 algebra of the pages (test infrastructure; see the package docstring).

[IntLoRA notes], section "1. AQS": W' = Q[W - sg(R)] + sg(R) + AB, so with the
base quantizer Q[x] = s * (W_round - z) the adapted weight is s*w + R* + AB.
Section "2. MLA": the same weight written multiplicatively,
W' = [s*I + (R + AB) / (W_round - z)] (.) (W_round - z), i.e. U (.) w with
U = s + (R + AB) / w, defined where w = W_round - z is non-zero.
Section "two implementation variants": MUL dequantizes as s_bar*(U_round - z_bar)(.)w,
SHIFT as sign(V)(.)(w >> shift) times the adaptation scale.
"""
from __future__ import annotations

import numpy as np


def signed_base(wround, z):
    """w = W_round - z as int64 (the pretrained integer term)."""
    return np.asarray(wround, np.int64) - np.asarray(z, np.int64)[:, None]


def additive_form(wround, z, s, rstar, A, B):
    """W' = s*w + R* + AB in binary64 (AQS form)."""
    w = signed_base(wround, z).astype(np.float64)
    AB = np.asarray(A, np.float64) @ np.asarray(B, np.float64)
    return np.asarray(s, np.float64)[:, None] * w + np.asarray(rstar, np.float64) + AB


def adaptation_fp64(wround, z, s, rstar, A, B):
    """U = s + (R* + AB) / w in binary64; NaN where w == 0."""
    w = signed_base(wround, z).astype(np.float64)
    AB = np.asarray(A, np.float64) @ np.asarray(B, np.float64)
    num = np.asarray(rstar, np.float64) + AB
    with np.errstate(divide="ignore", invalid="ignore"):
        U = np.asarray(s, np.float64)[:, None] + num / w
    U[w == 0] = np.nan
    return U


def multiplicative_form(wround, z, s, rstar, A, B):
    """W' = U (.) w in binary64 (MLA form); NaN where w == 0."""
    w = signed_base(wround, z).astype(np.float64)
    return adaptation_fp64(wround, z, s, rstar, A, B) * w


def dequant_mul(sbar, m):
    """Merged MUL weight s_bar * m (m = (U_round - z_bar) * w)."""
    return np.asarray(sbar, np.float64)[:, None] * np.asarray(m, np.float64)


def dequant_shift(sbar, m):
    """Merged SHIFT weight s_bar * m (m = sign(V) * (w >> shift))."""
    return np.asarray(sbar, np.float64)[:, None] * np.asarray(m, np.float64)


def ste_backward(wround, z, A, B, G):
    """Straight-through backward of the MUL / SHIFT fake-quant merge to the LoRA factors,
    in binary64 ([IntLoRA notes], "two implementation variants": training uses the STE).

    Reading: the rounding of U (MUL) and of log2|V| (SHIFT) pass gradients unchanged,
    s_bar and z_bar are constants, and R* takes none (sg(R), "1. AQS").  Then the merged
    weight behaves as U (.) w = s*w + R* + AB where w != 0, and is the constant 0 where
    w == 0, so with G = dL/dW' and the mask M = [w != 0]:
        dL/d(AB) = G (.) M,   dA = (G (.) M) B^T,   dB = A^T (G (.) M).
    Returns (dA, dB) as float64."""
    D = np.asarray(G, np.float64) * (signed_base(wround, z) != 0)
    return D @ np.asarray(B, np.float64).T, np.asarray(A, np.float64).T @ D
