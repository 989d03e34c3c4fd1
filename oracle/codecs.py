"""bf16 and FP8 e4m3fn codecs (oracle; test infrastructure only).

Formats, from the "ZYFA" README, Supported configurations: inputs are BF16,
or FP8 e4m3 as torch.float8_e4m3fn with 4 exponent and 3 mantissa bits;
the Kernel design list says every conversion rounds to nearest even.

e4m3fn (the OCP "fn" variant: finite, no infinities):
  sign bit, 4-bit exponent with bias 7, 3-bit mantissa.
  exponent field 0           -> subnormal: mantissa * 2^-9
  exponent field 1..15       -> (1 + mantissa/8) * 2^(e - 7)
  exponent 15, mantissa 7    -> NaN (0x7F / 0xFF); largest finite is 448.
The README's own facts follow from this: normals start at 2^-6, values
below 2^-10 round to zero, and the code of a positive number grows by 8
each time the value doubles (Kernel design, lean P).

bf16: the top 16 bits of an IEEE float32; encoding rounds the float32
value to nearest, ties to even mantissa.

All encoders here are exact: they work on integers or on float64 values
that represent every candidate exactly.
"""
from __future__ import annotations

import numpy as np

E4M3FN_MAX = 448.0


def _e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 codes as float64 (NaN for 0x7F, 0xFF)."""
    codes = np.arange(256, dtype=np.int64)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * mag
    val[(e == 15) & (m == 7)] = np.nan
    return val


_E4M3_TABLE = _e4m3fn_table()
# Non-negative finite values, codes 0x00..0x7E, strictly increasing.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = _E4M3_TABLE[:0x7F]


def e4m3fn_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values."""
    c = np.asarray(codes).astype(np.uint8)
    return _E4M3_TABLE[c.astype(np.int64)]


def e4m3fn_encode(x) -> np.ndarray:
    """float -> uint8 e4m3fn codes, round to nearest, ties to even code.

    Magnitudes above 448 saturate to 448 (the quantizer in this package never
    produces them); NaN maps to 0x7F. Negative zero keeps its sign bit.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a_c = np.minimum(a, E4M3FN_MAX)
    # index of the largest table value <= a
    hi = np.searchsorted(_POS_VALS, a_c, side="right")
    lo_idx = np.clip(hi - 1, 0, 0x7E)
    hi_idx = np.clip(hi, 0, 0x7E)
    lo_v = _POS_VALS[lo_idx]
    hi_v = _POS_VALS[hi_idx]
    d_lo = a_c - lo_v
    d_hi = hi_v - a_c
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_idx != lo_idx) & ((hi_idx & 1) == 0))
    code = np.where(pick_hi, hi_idx, lo_idx).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def bf16_encode_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.

    Finite inputs only (NaN payloads are not specified by the pages).
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    return (rounded & 0xFFFF).astype(np.uint16)


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """float32 -> float64 value of its bf16 rounding."""
    return bf16_decode(bf16_encode_bits(x))
