"""Pins of the FP8 probability-rounding model (tests/fp8_rounding_model.py),
CPU only.

Each check rests on something other than the oracle itself: hand-computed
e4m3fn weights (tests/golden/fp8_rounding_worked.txt), the exact softmax definition
in the cases where rounding is exact (integer base-2 scores), closed forms of
weighted averages, and the mean of the piecewise-linear 2^y.
"""
import math
import os

import numpy as np
import pytest

from oracle import causal_attention_rows_ref, e4m3fn_decode
import fp8_rounding_model as fp8_p

GOLD = os.path.join(os.path.dirname(__file__), "golden")
LN2 = math.log(2.0)


def _worked():
    rows = []
    with open(os.path.join(GOLD, "fp8_rounding_worked.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            mode, y, code, w = line.split()
            rows.append((mode, float(y), int(code, 16), float(w)))
    return rows


@pytest.mark.parametrize("mode,y,code,w", _worked())
def test_worked_codes(mode, y, code, w):
    c = (fp8_p.lean_code if mode == "lean" else fp8_p.exact_code)(np.array([y]))[0]
    assert c == code
    if mode == "precise":
        assert fp8_p.precise_value(np.array([y]))[0] == w
    else:
        assert e4m3fn_decode(np.array([c], np.uint8))[0] == w


def test_precise_value_error_bound():
    # hi carries 4 significant bits (error <= 2^-4 relative); lo rounds the
    # remainder to 4 more, so |hi + lo - p| <= 2^-4 * 2^-4 * p for p in the
    # normal range of e4m3 (p >= 2^-2 keeps the remainder normal too)
    rng = np.random.default_rng(8)
    y = rng.uniform(-2.0, 0.999, 100000)
    p = np.exp2(y)
    r = np.abs(fp8_p.precise_value(y) - p) / p
    assert r.max() <= 2.0 ** -8
    hi = e4m3fn_decode(fp8_p.exact_code(y).astype(np.uint8))
    assert (np.abs(hi - p) / p).max() > 2.0 ** -6   # hi alone is much coarser


def test_lean_constant_rounds_integers_to_the_exact_code():
    y = np.arange(-6, 2)
    assert np.array_equal(fp8_p.lean_code(y), 8 * y + 56)
    assert np.array_equal(fp8_p.lean_code(y), fp8_p.exact_code(y))


def test_lean_is_unbiased_and_bounded():
    # mean ratio of the lean value to 2^y over uniform fractional parts is 1
    # (the constant removes the factor 1/(2 ln(2)^2) of the linear
    # interpolation); the ratio stays within the interpolation's 6.2% and
    # half a code step (2^(+-1/16)) around that.
    rng = np.random.default_rng(3)
    y = rng.uniform(-5.0, 0.0, 200000)
    r = e4m3fn_decode(fp8_p.lean_code(y).astype(np.uint8)) / np.exp2(y)
    assert abs(r.mean() - 1.0) < 2e-3
    c = 1.0 / (2 * LN2 ** 2)
    assert r.min() >= 2.0 ** (-1 / 16) / c - 1e-12
    assert r.max() <= 2.0 ** (1 / 16) * 1.0615 / c
    assert r.min() < 0.95 and r.max() > 1.03


@pytest.mark.parametrize("p_mode", fp8_p.P_MODES)
def test_integer_scores_reduce_to_exact_softmax(p_mode):
    # base-2 scores that are integers in [-2, 2], so within 4 binades of
    # their block's largest: every rounding is exact, so the result is exact
    # softmax
    rng = np.random.default_rng(7)
    S, d = 300, 2
    q = rng.integers(-1, 2, (1, S, 1, d)).astype(np.float64)
    k = rng.integers(-1, 2, (1, S, 1, d)).astype(np.float64)
    v = rng.standard_normal((1, S, 1, 16))
    rows = np.arange(S)
    o1, l1 = fp8_p.fp8_attention_rows_ref(q, k, v, 0, 0, rows, softmax_scale=LN2, p_mode=p_mode)
    o2, l2 = causal_attention_rows_ref(q, k, v, 0, 0, rows, softmax_scale=LN2)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def _row(xvals, i, p_mode):
    w, m = fp8_p.row_weights(np.asarray(xvals, dtype=np.float64), i, p_mode)
    return w * 2.0 ** m


def test_two_key_row_weights():
    # row 1 with base-2 scores (0, -0.5): weights (1, 0.6875) exact and
    # (1, 0.75) lean; in lean_offdiag both keys are on the diagonal tile
    assert np.array_equal(_row([0.0, -0.5], 1, "exact"), [1.0, 0.6875])
    assert np.array_equal(_row([0.0, -0.5], 1, "lean"), [1.0, 0.75])
    assert np.array_equal(_row([0.0, -0.5], 1, "lean_offdiag"), [1.0, 0.6875])


def test_block_power_of_two():
    # a block whose largest score is 3.5 below the reference: e_b = -4, the
    # block is coded around 2^0.5 and multiplied back by 2^-4
    x = np.full(64, -200.0)
    x[0] = 0.0
    x[32] = -3.5
    w = _row(x, 63, "exact")
    assert w[0] == 1.0 and w[32] == 1.375 * 2.0 ** -4
    assert np.all(w[1:32] == 0) and np.all(w[33:] == 0)
    w = _row(x, 63, "lean")
    assert w[32] == 1.5 * 2.0 ** -4


def test_subnormal_and_underflow_weights():
    assert np.array_equal(_row([0.0, -9.5], 1, "exact"), [1.0, 2.0 ** -9])
    assert np.array_equal(_row([0.0, -7.0, -6.5], 2, "lean"), [1.0, 0.0, 2.0 ** -7])


def test_query_tile_is_exact_in_lean_offdiag():
    # row 384 lies in query tile 1 (rows 256..511): key tiles 2 and 3 (keys
    # 256..) take exact P, key tiles 0 and 1 lean P; all four marked keys are
    # half a binade below the reference
    x = np.full(385, -300.0)
    x[0] = 0.0
    x[[1, 200, 300, 384]] = -0.5
    w = _row(x, 384, "lean_offdiag")
    assert w[0] == 1.0 and w[1] == 0.75                 # lean, key tile 0
    assert w[200] == 1.5 * 2.0 ** -1                    # lean, key tile 1 (block e_b = -1)
    assert w[300] == 1.375 * 2.0 ** -1                  # exact, key tile 2: RNE(2^0.5)
    assert w[384] == 1.375 * 2.0 ** -1                  # exact, key tile 3
    w = _row(x, 384, "lean")
    assert w[300] == 1.5 * 2.0 ** -1 and w[384] == 1.5 * 2.0 ** -1
    # row 255 lies in query tile 0: every key is exact
    assert np.array_equal(_row(x[:256], 255, "lean_offdiag"), _row(x[:256], 255, "exact"))


def test_query_tile_of_128_rows_in_lean_offdiag():
    # with 128-row query tiles, row 200 lies in query tile 1 (rows 128..255):
    # key tile 1 (keys 128..) takes exact P and key tile 0 lean P; with
    # 256-row query tiles both are exact
    x = np.full(201, -300.0)
    x[0] = 0.0
    x[[1, 130, 200]] = -0.5
    w = fp8_p.row_weights(x, 200, "lean_offdiag", query_tile=128)[0]
    assert w[0] == 1.0 and w[1] == 0.75                 # lean, key tile 0
    assert w[130] == 1.375 * 2.0 ** -1                  # exact, key tile 1: RNE(2^0.5)
    assert w[200] == 1.375 * 2.0 ** -1
    w = fp8_p.row_weights(x, 200, "lean_offdiag", query_tile=256)[0]
    assert w[1] == 1.375 * 2.0 ** -1                    # exact: row 200 is in the first 256-row tile
    # rows of the first 128-row query tile: every key is exact
    assert np.array_equal(fp8_p.row_weights(x[:128], 127, "lean_offdiag", query_tile=128)[0],
                          fp8_p.row_weights(x[:128], 127, "exact")[0])


def test_lazy_reference():
    # tile 0 peaks at 0.5; tile 1 peaks at 1.0, within the threshold, so the
    # reference stays at 0.5 and key 128 is coded at y = 0.5 (lean: 1.5)
    x = np.full(200, -300.0)
    x[0], x[128] = 0.5, 1.0
    w = _row(x, 199, "lean")
    assert w[0] == 2.0 ** 0.5 and w[128] == 1.5 * 2.0 ** 0.5
    # a tile peak beyond the threshold moves the reference: key 128 is coded
    # at y = 0 and key 0 keeps its tile-0 weight
    x[128] = 10.0
    w = _row(x, 199, "lean")
    assert w[0] == 2.0 ** 0.5 and w[128] == 2.0 ** 10


@pytest.mark.parametrize("p_mode", fp8_p.P_MODES)
def test_row0_and_constant_keys(p_mode):
    rng = np.random.default_rng(11)
    S, d = 260, 8
    q = rng.standard_normal((1, S, 1, d))
    k = np.tile(rng.standard_normal((1, 1, 1, d)), (1, S, 1, 1))
    v = rng.standard_normal((1, S, 1, 8))
    rows = np.arange(S)
    o, _ = fp8_p.fp8_attention_rows_ref(q, k, v, 0, 0, rows, p_mode=p_mode)
    np.testing.assert_allclose(o[0], v[0, 0, 0], rtol=0, atol=1e-15)
    prefix = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(o, prefix, rtol=0, atol=1e-12)


def test_lean_offdiag_equals_exact_within_first_query_tile():
    rng = np.random.default_rng(5)
    S, d = 256, 16
    q, k, v = (rng.standard_normal((1, S, 1, d)) for _ in range(3))
    rows = np.arange(S)
    a = fp8_p.fp8_attention_rows_ref(q, k, v, 0, 0, rows, p_mode="exact")
    b = fp8_p.fp8_attention_rows_ref(q, k, v, 0, 0, rows, p_mode="lean_offdiag")
    c = fp8_p.fp8_attention_rows_ref(q, k, v, 0, 0, rows, p_mode="lean")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])


def test_rounded_modes_stay_near_exact_softmax():
    # the rounded probabilities change the result by at most a few percent
    # of V's spread (e4m3 keeps 3 mantissa bits)
    rng = np.random.default_rng(9)
    S, d = 384, 32
    q, k, v = (rng.standard_normal((1, S, 1, d)) for _ in range(3))
    rows = np.arange(S)
    ref = causal_attention_rows_ref(q, k, v, 0, 0, rows, softmax_scale=1 / math.sqrt(d))
    for p_mode in fp8_p.P_MODES:
        o, l = fp8_p.fp8_attention_rows_ref(q, k, v, 0, 0, rows, p_mode=p_mode)
        assert np.abs(o - ref[0]).max() < 0.15
        assert np.abs(o - ref[0]).mean() < 6e-3
        assert np.abs(l - ref[1]).max() < 0.06
