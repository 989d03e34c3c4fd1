"""Model of this library's FP8 probability rounding (float64; a regression
check of the FP8 kernels, not an oracle).

The oracle (oracle/attention.py) is exact softmax attention on the
dequantized inputs, and every FP8 accuracy claim is made against it. An FP8
kernel instead weights V by e4m3fn-rounded probabilities and normalises by
the total of those rounded weights. This module writes out which rounded
values THIS library's kernels use, so a GPU result can be checked far more
tightly than the accuracy gate allows. Its constants are the kernels'
choices, not the pages': 128-key tiles, 32-key scale blocks (the scaled
MFMA's block; the "ZYFA" README uses 64 keys), a lazy-rescale threshold of
8 base-2 units (the README names 0.125 in FP8) and exact P on the key tiles
of a 256-row query block (the README uses lean P throughout at d = 128).
It follows the README's Kernel design section for the steps themselves
(lazy rescaling; per-block scaling; lean P; row sum on the matrix unit) and
its Accuracy section (the output is a weighted average whose weights are the
rounded probabilities, and the LSE comes from them).

For query row i (keys j <= i), with x_j = softmax_scale * log2(e) *
<q_i, k_j> the score in base-2 units:

1. Keys are visited in ascending tiles of KEY_TILE keys. The row keeps a
   running reference m (-inf before the first tile). At each tile, with M
   the largest x_j of the tile, m becomes M if M > m + TAU, else stays:
   the lazy rescale. (The README rescales when the running maximum grows by
   more than a threshold; TAU = 8 base-2 units is this implementation's
   threshold.)
2. Within a tile, each block of BLOCK consecutive keys (block index j //
   BLOCK) gets the power of two 2^e_b with e_b = floor(B_b - m), B_b the
   block's largest x_j (at least 2^-126, the smallest normal float32): the
   block's largest probability 2^(B_b - m) divided by 2^e_b lies in [1, 2).
3. Each key gets an e4m3fn code c_j for y_j = x_j - m - e_b:
   - exact P: c_j = RNE_e4m3fn(2^y_j);
   - lean P:  c_j = clamp(RNE(8 y_j + LEAN_C), 0, 255), the code read as an
     integer (it grows by 8 per doubling, so 8 y + 56 is the code of 2^y at
     integer y and interpolates linearly in between; LEAN_C = 56 +
     8 log2(2 ln(2)^2) = 55.54 instead of 56 makes the piecewise-linear
     value 2^floor(y) (1 + frac(y)) unbiased: its mean ratio to 2^y over a
     uniform frac(y) is 1 / (2 ln(2)^2));
   - precise ("precise"): two codes per key, hi = RNE_e4m3fn(2^y) and
     lo = RNE_e4m3fn(2^y - value(hi)), whose values add (the library's
     precise mode multiplies both into V with the block's scale);
   - lean P off the diagonal query tile ("lean_offdiag"): the query rows
     are grouped in blocks of query_tile rows (256, which the kernels use
     at every query-tile height); keys of the key tiles that hold the rows
     of row i's own query tile (key tile t >= floor(i / query_tile) *
     query_tile / KEY_TILE) get exact P, which covers every key of the rows
     with the fewest keys; the key tiles before them get lean P. (Which tiles keep exact P is this
     implementation's choice; the README uses lean P throughout at d = 128.)
4. The key's weight is w_j = value(c_j) * 2^(e_b + m) (precise: the sum of
   the two values), with m the reference
   when its tile was visited. O_i = sum_j w_j v_j / sum_j w_j and
   LSE_i = ln(sum_j w_j).

All weights are formed relative to the row's final reference (an exact
power of two, added back to the LSE), so float64 never overflows.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from oracle.attention import _split, kv_head
from oracle.codecs import e4m3fn_decode, e4m3fn_encode

KEY_TILE = 128
QUERY_TILE = 256
BLOCK = 32
TAU = 8.0
LOG2E = 1.4426950408889634073599246810019
LEAN_C = 56.0 + 8.0 * math.log2(2.0 * math.log(2.0) ** 2)
P_MODES = ("exact", "lean", "lean_offdiag", "precise")


def lean_code(y) -> np.ndarray:
    """Lean-P code of 2^y (y in base-2 units), clamped to 0..255."""
    y = np.asarray(y, dtype=np.float64)
    return np.clip(np.rint(8.0 * y + LEAN_C), 0, 255).astype(np.int64)


def exact_code(y) -> np.ndarray:
    """RNE e4m3fn code of 2^y."""
    return e4m3fn_encode(np.exp2(np.asarray(y, dtype=np.float64))).astype(np.int64)


def precise_value(y) -> np.ndarray:
    """value(hi) + value(lo) of the precise mode for p = 2^y."""
    p = np.exp2(np.asarray(y, dtype=np.float64))
    hi = e4m3fn_decode(e4m3fn_encode(p))
    return hi + e4m3fn_decode(e4m3fn_encode(p - hi))


def row_weights(x: np.ndarray, i: int, p_mode: str, *, key_tile: int = KEY_TILE, block: int = BLOCK,
                tau: float = TAU, query_tile: int = QUERY_TILE):
    """Weights of keys 0..i of one row (x holds their base-2 scores), divided
    by 2^m_final, and m_final. Returns (w, m_final)."""
    if p_mode not in P_MODES:
        raise ValueError(f"p_mode must be one of {P_MODES}")
    if key_tile % block:
        raise ValueError("key_tile must be a multiple of block")
    x = np.asarray(x, dtype=np.float64)
    n = i + 1
    assert x.shape[0] == n
    m = -np.inf
    exps = np.zeros(n)     # e_b + m_t per key
    codes = np.zeros(n, dtype=np.int64)
    vals = np.zeros(n)     # precise mode: value(hi) + value(lo)
    diag_tile = i // key_tile
    exact_from = (i // query_tile) * query_tile // key_tile
    for t in range(diag_tile + 1):
        lo, hi = t * key_tile, min((t + 1) * key_tile, n)
        mt = x[lo:hi].max()
        if mt > m + tau:
            m = mt
        for b0 in range(lo, hi, block):
            b1 = min(b0 + block, hi)
            e_b = max(math.floor(x[b0:b1].max() - m), -126)
            y = x[b0:b1] - m - e_b
            lean = p_mode == "lean" or (p_mode == "lean_offdiag" and t < exact_from)
            if p_mode == "precise":
                vals[b0:b1] = precise_value(y)
            else:
                codes[b0:b1] = lean_code(y) if lean else exact_code(y)
            exps[b0:b1] = e_b + m
    m_final = m
    if p_mode != "precise":
        vals = e4m3fn_decode(codes.astype(np.uint8))
    w = vals * np.exp2(exps - m_final)
    return w, m_final


def fp8_attention_rows_ref(q, k, v, b: int, h: int, rows, *, layout: str = "bshd",
                           softmax_scale: Optional[float] = None, p_mode: str = "exact",
                           key_tile: int = KEY_TILE, block: int = BLOCK, tau: float = TAU,
                           query_tile: int = QUERY_TILE):
    """O (len(rows), d_v) and natural-log LSE (len(rows),) of the given query
    rows of batch b and query head h, with probabilities rounded as above.
    q, k, v are the dequantized inputs (code value times descale)."""
    qs, ks, vs = (_split(np.asarray(t), layout) for t in (q, k, v))
    nheads, nheads_k, d_qk = qs.shape[1], ks.shape[1], qs.shape[3]
    scale = (1.0 / math.sqrt(d_qk)) if softmax_scale is None else float(softmax_scale)
    hk = kv_head(h, nheads, nheads_k)
    qh = np.asarray(qs[b, h], dtype=np.float64)
    kh = np.asarray(ks[b, hk], dtype=np.float64)
    vh = np.asarray(vs[b, hk], dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], vh.shape[1]))
    lse = np.zeros(rows.shape[0])
    for r, i in enumerate(rows):
        x = (scale * LOG2E) * (kh[: i + 1] @ qh[i])
        w, m = row_weights(x, int(i), p_mode, key_tile=key_tile, block=block, tau=tau, query_tile=query_tile)
        l = w.sum()
        out[r] = (w @ vh[: i + 1]) / l
        lse[r] = (math.log2(l) + m) * math.log(2.0)
    return out, lse
