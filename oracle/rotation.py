"""Orthogonal rotation of q and k before FP8 quantization, in float64
(oracle; test infrastructure only).

"ZYFA" README, "Using FP8 attention in a model": q and k are multiplied by
an orthogonal matrix R before quantization, so (q R)(k R)^T = q k^T and only
the rounding error changes; R = diag(s) H / sqrt(d) with H the Hadamard
matrix of Sylvester's construction (H_1 = [1], H_2n = [[H_n, H_n], [H_n,
-H_n]]) and s a vector of random signs, for d a power of two (the library
rotates d = 128).

Readings:
- The signs are an input (one +1 / -1 per channel).
- Quantization of the rotated tensor follows quantize.fp8_quantize_ref: one
  power-of-two scale per tensor, round to nearest even.
"""
from __future__ import annotations

import numpy as np

from .quantize import fp8_quantize_ref


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_matrix(d: int, signs) -> np.ndarray:
    """R (d x d) for d a power of two (128 in the library)."""
    s = np.asarray(signs, dtype=np.float64)
    if s.shape != (d,) or not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be d values of +1 or -1")
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    return s[:, None] * (hadamard(d) / np.sqrt(d))


def rotate_ref(x, signs) -> np.ndarray:
    """x (..., d) -> x R in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x @ rotation_matrix(x.shape[-1], signs)


def quantize_rotated_ref(x, signs):
    """(codes, descale, rotated values): fp8_quantize_ref of x R."""
    y = rotate_ref(x, signs)
    codes, d = fp8_quantize_ref(y)
    return codes, d, y


# ---- K smoothing ("ZYFA" README, "Using FP8 attention in a model"):
# before the rotation, take from every key of a head that head's average
# key over all positions.
# Every key of a row then loses the same vector c, so each score of the row
# moves by the same q . c and the softmax, hence the output, is unchanged;
# the log-sum-exp moves by scale * q . c.

def key_mean_ref(k, layout: str = "bshd") -> np.ndarray:
    """k (B, S, Hk, d) or (B, Hk, S, d) -> mean over positions, (B, Hk, d), float64."""
    k = np.asarray(k, dtype=np.float64)
    return k.mean(axis=1 if layout == "bshd" else 2)


def quantize_shifted_rotated_ref(x, shift, signs, layout: str = "bshd"):
    """(codes, descale, rotated values) of (x - shift[b, h]) R, quantized per
    tensor; shift (B, H, d) is subtracted from every position of its head."""
    x = np.asarray(x, dtype=np.float64)
    sh = np.asarray(shift, dtype=np.float64)
    sh = sh[:, None, :, :] if layout == "bshd" else sh[:, :, None, :]
    return quantize_rotated_ref(x - sh, signs)
