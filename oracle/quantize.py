"""Power-of-two per-tensor FP8 quantization (oracle; test infrastructure only).

"ZYFA" README, Usage: fp8_quantize gives one power-of-two scale per tensor
and returns the descale (the factor that maps the FP8 tensor back to its
original range). The workload text fixes the target: the tensor's largest
magnitude maps at most to 448, the e4m3fn maximum. The plainest reading that
never saturates is

    amax    = max |x| over the whole tensor
    descale = 2^ceil(log2(amax / 448))     (descale = 1 when amax == 0)
    code    = e4m3fn_RNE(x / descale)

The README also requires a tensor descale to be a positive normal float32
(Usage), so the descale is never below 2^-126 (it only matters for tensors
whose largest magnitude is below 448 * 2^-127).

x / descale is exact (a power of two), so each code is one RNE rounding
(Kernel design: every conversion rounds to nearest even).
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import E4M3FN_MAX, e4m3fn_encode


def pow2_descale(amax: float) -> float:
    """Smallest power of two d with amax / d <= 448 (1 for amax == 0).

    Found by exact comparisons of amax with 448 * 2^e in float64 (both sides
    are exact there), starting from a log2 estimate.
    """
    if amax == 0.0:
        return 1.0
    e = math.ceil(math.log2(amax / E4M3FN_MAX))
    while math.ldexp(E4M3FN_MAX, e) < amax:
        e += 1
    while math.ldexp(E4M3FN_MAX, e - 1) >= amax:
        e -= 1
    return math.ldexp(1.0, max(e, -126))


def fp8_quantize_ref(x):
    """x (float values, e.g. bf16-decoded) -> (uint8 codes, float32 descale)."""
    x = np.asarray(x, dtype=np.float64)
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    d = pow2_descale(amax)
    codes = e4m3fn_encode(x / d)
    return codes, np.float32(d)
