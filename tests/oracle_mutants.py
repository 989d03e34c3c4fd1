"""Planted mistakes in the oracle, for tests/test_oracle_mutants.py.

Each mutant replaces one small function (or table) of oracle/ with a copy
that carries one plausible mistake: a dropped term, a wrong sign, index or
axis, a transposed operand, an off-by-one mask, a wrong rounding rule. The
pins of the oracle (tests/test_oracle_*.py) must fail on every one of them:
a pin set that a plausible mistake passes does not pin the oracle.

A mutant is applied inside a separate pytest process (ZYFA_ORACLE_MUTANT
names it; tests/conftest.py calls apply()), so the oracle of every other
test is never touched. Nothing here is used by the library.
"""
from __future__ import annotations

import math
import types

import numpy as np

import oracle
import oracle.attention as att
import oracle.codecs as codecs
import oracle.partial as partial
import oracle.quantize as quantize
import oracle.rotation as rotation


def _head_rows(kind):
    """oracle.attention._head_rows with one planted mistake."""
    def f(qh, kh, vh, scale, rows):
        rows = np.asarray(rows, dtype=np.int64)
        if kind == "scores_transposed":
            sc = scale * (kh[rows] @ qh.T)
        else:
            sc = scale * (qh[rows] @ kh.T)
        keys = np.arange(kh.shape[0], dtype=np.int64)
        if kind == "mask_excludes_diagonal":
            sc[keys[None, :] >= rows[:, None]] = -np.inf
        elif kind == "mask_admits_next_key":
            sc[keys[None, :] > rows[:, None] + 1] = -np.inf
        elif kind != "no_causal_mask":
            sc[keys[None, :] > rows[:, None]] = -np.inf
        m = sc.max(axis=1, keepdims=True)
        p = np.exp(sc) if kind == "no_max_subtraction" else np.exp(sc - m)
        l = p.sum(axis=1, keepdims=True)
        v = np.roll(vh, 1, axis=0) if kind == "v_rows_shifted" else vh
        o = p @ v if kind == "output_not_normalised" else (p @ v) / l
        if kind == "lse_log2":
            lse = (m[:, 0] + np.log(l[:, 0])) / math.log(2.0)
        elif kind in ("lse_drops_max", "no_max_subtraction"):
            lse = np.log(l[:, 0])
        else:
            lse = m[:, 0] + np.log(l[:, 0])
        return o, lse
    return f


def _causal_probs_unmasked(qh, kh, scale):
    qh, kh = np.asarray(qh, dtype=np.float64), np.asarray(kh, dtype=np.float64)
    p = np.exp(scale * (qh @ kh.T))
    return p / p.sum(axis=1, keepdims=True)


class _NumpyWithSqrt(types.ModuleType):
    """numpy, except sqrt: the default scale becomes 1/d instead of 1/sqrt(d)."""
    def __init__(self):
        super().__init__("numpy_mutant")

    def __getattr__(self, name):
        return getattr(np, name)

    @staticmethod
    def sqrt(x):
        return np.asarray(x, dtype=np.float64)


def _split_never_swaps(x, layout):
    if layout not in ("bshd", "bhsd"):
        raise ValueError(layout)
    return x


def _range_head_strict(qh, kh, vh, scale, rows, q_pos0, k_pos0):
    """oracle.partial._range_head with a key at the query's own position hidden."""
    rows = np.asarray(rows, dtype=np.int64)
    if kh.shape[0] == 0:
        return np.zeros((len(rows), vh.shape[1])), np.full(len(rows), -np.inf)
    sc = scale * (qh[rows] @ kh.T)
    kpos = k_pos0 + np.arange(kh.shape[0], dtype=np.int64)
    qpos = q_pos0 + rows
    sc[kpos[None, :] >= qpos[:, None]] = -np.inf
    m = sc.max(axis=1, keepdims=True)
    seen = np.isfinite(m[:, 0])
    m[~seen] = 0.0
    p = np.exp(sc - m)
    l = p.sum(axis=1, keepdims=True)
    o = np.zeros((len(rows), vh.shape[1]))
    o[seen] = (p[seen] @ vh) / l[seen]
    lse = np.full(len(rows), -np.inf)
    lse[seen] = m[seen, 0] + np.log(l[seen, 0])
    return o, lse


def _range_head_empty_lse_zero(qh, kh, vh, scale, rows, q_pos0, k_pos0):
    o, lse = _ORIG["range_head"](qh, kh, vh, scale, rows, q_pos0, k_pos0)
    return o, np.where(np.isneginf(lse), 0.0, lse)


def _merge(kind):
    def f(o_a, lse_a, o_b, lse_b):
        o_a, o_b = np.asarray(o_a, dtype=np.float64), np.asarray(o_b, dtype=np.float64)
        la, lb = np.asarray(lse_a, dtype=np.float64), np.asarray(lse_b, dtype=np.float64)
        m = np.maximum(la, lb)
        empty = ~np.isfinite(m)
        ms = np.where(empty, 0.0, m)
        wa, wb = np.exp(la - ms), np.exp(lb - ms)
        tot = wa + wb
        if kind == "merge_lse_is_max":
            lse = m
        else:
            lse = np.where(empty, -np.inf, ms + np.log(np.where(empty, 1.0, tot)))
        den = np.where(empty, 1.0, tot)
        if kind == "merge_weights_swapped":
            wa, wb = wb, wa
        o = (wa / den)[..., None] * o_a + (wb / den)[..., None] * o_b
        return o, lse
    return f


def _e4m3_table_bias8():
    codes = np.arange(256, dtype=np.int64)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    val = sign * mag
    val[(e == 15) & (m == 7)] = np.nan
    return val


def _e4m3_encode_ties_up(x):
    """e4m3fn_encode with ties rounded away from zero instead of to even."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), codecs.E4M3FN_MAX)
    pos = codecs._POS_VALS
    hi = np.searchsorted(pos, a, side="right")
    lo_idx = np.clip(hi - 1, 0, 0x7E)
    hi_idx = np.clip(hi, 0, 0x7E)
    pick_hi = (pos[hi_idx] - a) <= (a - pos[lo_idx])
    code = np.where(pick_hi, hi_idx, lo_idx).astype(np.int64)
    code = code | np.where(np.signbit(x), 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def _bf16_truncate(x):
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _descale(kind):
    def f(amax):
        if amax == 0.0:
            return 1.0
        if kind == "descale_floor":
            return math.ldexp(1.0, max(math.floor(math.log2(amax / codecs.E4M3FN_MAX)), -126))
        e = math.ceil(math.log2(amax / codecs.E4M3FN_MAX))
        while math.ldexp(codecs.E4M3FN_MAX, e) < amax:
            e += 1
        while math.ldexp(codecs.E4M3FN_MAX, e - 1) >= amax:
            e -= 1
        return math.ldexp(1.0, e)              # descale_no_floor: no 2^-126 minimum
    return f


def _rotation(kind):
    def f(d, signs):
        s = np.asarray(signs, dtype=np.float64)
        if s.shape != (d,) or not np.all(np.abs(s) == 1.0):
            raise ValueError("signs must be d values of +1 or -1")
        if d < 1 or d & (d - 1):
            raise ValueError("d must be a power of two")
        h = rotation.hadamard(d)
        if kind == "signs_on_columns":
            return h * s[None, :] / np.sqrt(d)
        return s[:, None] * h                   # hadamard_unnormalised
    return f


def _key_mean_wrong_axis(k, layout="bshd"):
    """The mean taken over the axis the other layout uses for positions."""
    k = np.asarray(k, dtype=np.float64)
    return k.mean(axis=2 if layout == "bshd" else 1)


_ORIG = {"range_head": partial._range_head}


def _set(pairs):
    for mod, name, value in pairs:
        setattr(mod, name, value)


MUTANTS = {
    # attention
    "mask_excludes_diagonal": lambda: _set([(att, "_head_rows", _head_rows("mask_excludes_diagonal"))]),
    "mask_admits_next_key": lambda: _set([(att, "_head_rows", _head_rows("mask_admits_next_key"))]),
    "no_causal_mask": lambda: _set([(att, "_head_rows", _head_rows("no_causal_mask")),
                                    (att, "causal_probs_ref", _causal_probs_unmasked),
                                    (oracle, "causal_probs_ref", _causal_probs_unmasked)]),
    "scores_transposed": lambda: _set([(att, "_head_rows", _head_rows("scores_transposed"))]),
    "no_max_subtraction": lambda: _set([(att, "_head_rows", _head_rows("no_max_subtraction"))]),
    "v_rows_shifted": lambda: _set([(att, "_head_rows", _head_rows("v_rows_shifted"))]),
    "output_not_normalised": lambda: _set([(att, "_head_rows", _head_rows("output_not_normalised"))]),
    "lse_log2": lambda: _set([(att, "_head_rows", _head_rows("lse_log2"))]),
    "lse_drops_max": lambda: _set([(att, "_head_rows", _head_rows("lse_drops_max"))]),
    "gqa_head_modulo": lambda: _set([(att, "kv_head", lambda h, nheads, nheads_k: h % nheads_k),
                                     (partial, "kv_head", lambda h, nheads, nheads_k: h % nheads_k)]),
    "default_scale_inverse_d": lambda: _set([(att, "np", _NumpyWithSqrt()), (partial, "np", _NumpyWithSqrt())]),
    "bshd_read_as_bhsd": lambda: _set([(att, "_split", _split_never_swaps), (partial, "_split", _split_never_swaps)]),
    # partial ranges and the merge
    "range_hides_own_position": lambda: _set([(partial, "_range_head", _range_head_strict)]),
    "range_empty_row_lse_zero": lambda: _set([(partial, "_range_head", _range_head_empty_lse_zero)]),
    "merge_lse_is_max": lambda: _set([(partial, "lse_merge_ref", _merge("merge_lse_is_max")),
                                      (oracle, "lse_merge_ref", _merge("merge_lse_is_max"))]),
    "merge_weights_swapped": lambda: _set([(partial, "lse_merge_ref", _merge("merge_weights_swapped")),
                                           (oracle, "lse_merge_ref", _merge("merge_weights_swapped"))]),
    # codecs and the quantizer
    "e4m3_exponent_bias_8": lambda: _set([(codecs, "_E4M3_TABLE", _e4m3_table_bias8()),
                                          (codecs, "_POS_VALS", _e4m3_table_bias8()[:0x7F])]),
    "e4m3_ties_away_from_zero": lambda: _set([(codecs, "e4m3fn_encode", _e4m3_encode_ties_up),
                                              (oracle, "e4m3fn_encode", _e4m3_encode_ties_up),
                                              (quantize, "e4m3fn_encode", _e4m3_encode_ties_up)]),
    "bf16_truncates": lambda: _set([(codecs, "bf16_encode_bits", _bf16_truncate),
                                    (oracle, "bf16_encode_bits", _bf16_truncate)]),
    "descale_floor": lambda: _set([(quantize, "pow2_descale", _descale("descale_floor"))]),
    "descale_no_floor": lambda: _set([(quantize, "pow2_descale", _descale("descale_no_floor"))]),
    # rotation
    "signs_on_columns": lambda: _set([(rotation, "rotation_matrix", _rotation("signs_on_columns")),
                                      (oracle, "rotation_matrix", _rotation("signs_on_columns"))]),
    "hadamard_unnormalised": lambda: _set([(rotation, "rotation_matrix", _rotation("hadamard_unnormalised")),
                                           (oracle, "rotation_matrix", _rotation("hadamard_unnormalised"))]),
    "key_mean_over_heads": lambda: _set([(rotation, "key_mean_ref", _key_mean_wrong_axis),
                                         (oracle, "key_mean_ref", _key_mean_wrong_axis)]),
}


def apply(name: str) -> None:
    MUTANTS[name]()
