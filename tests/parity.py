"""Helpers shared by the GPU parity tests: input staging and tolerances.

Both sides see the same inputs: the seeded float32 draws of `workloads`
are cast to bf16 by torch for the GPU and by the oracle's own codec for the
oracle; `bf16_pair` checks that the two casts agree bit for bit.
"""
import math

import numpy as np
import torch

import oracle

# BF16 gate: max |d out| <= 1e-2 and |d LSE| <= 1e-3. The output is bf16, so
# an exactly computed result still carries up to half an ulp of rounding,
# 2^-8 |ref| (over 1e-2 once |ref| >= 2.56); the element bound adds exactly
# that allowance. The literal max is reported beside it.
BF16_OUT_ABS = 1e-2
BF16_OUT_REL_ROUND = 2.0 ** -8
BF16_LSE_ABS = 1e-3
# FP8 gate (oracle on the dequantized inputs): max <= 6e-2, mean <= 5e-3,
# with the same bf16 output-rounding allowance on the max.
FP8_OUT_MAX = 6e-2
FP8_OUT_MEAN = 5e-3
# FP8 LSE (from the rounded probabilities): each weight is off by at most
# 2^-4 relative (one e4m3 rounding), so the row sum's log by < 0.065 nats;
# the precise mode keeps 2^-8 (hi + lo), i.e. < 0.004 nats, gated at 0.008.
FP8_LSE_MAX = 0.065
FP8_PRECISE_LSE_MAX = 0.008


def bf16_pair(x: np.ndarray, device="cuda"):
    """(torch bf16 CUDA tensor, float64 values the oracle uses)."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    ref = oracle.bf16_round(x)
    bits_torch = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits_torch, oracle.bf16_encode_bits(x)), "bf16 casts disagree"
    return t.to(device), ref


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def score_magnitude(qh: np.ndarray, kh: np.ndarray, scale: float, rows) -> np.ndarray:
    """scale * max_{j <= i} sum_c |q_ic k_jc| for the given rows of one head:
    the size of the terms an fp32 score accumulation rounds."""
    rows = np.asarray(rows)
    a = np.abs(qh[rows]) @ np.abs(kh[: int(rows.max()) + 1]).T
    a[np.arange(a.shape[1])[None, :] > rows[:, None]] = 0.0
    return scale * a.max(axis=1)


# fp32 score accumulation (MFMA, d_qk terms) rounds at about 2^-24 of the term
# magnitude per step; 2^-20 of it is the LSE allowance added on rows whose
# scores are large (activation-like inputs). On N(0, 1) inputs it is < 1e-5.
LSE_ROUND_REL = 2.0 ** -20


def check_bf16(out, ref_out, lse=None, ref_lse=None, what="", lse_mag=None):
    d = np.abs(out - ref_out)
    bound = BF16_OUT_ABS + BF16_OUT_REL_ROUND * np.abs(ref_out)
    worst = np.unravel_index(np.argmax(d - bound), d.shape)
    msg = f"{what}: max|dout|={d.max():.3e} mean={d.mean():.2e} worst at {worst} (ref {ref_out[worst]:.4f} got {out[worst]:.4f})"
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    assert np.all(d <= bound), msg
    if lse is not None:
        dl = np.abs(lse - ref_lse)
        assert np.all(np.isfinite(lse)), what + ": non-finite lse"
        allow = BF16_LSE_ABS if lse_mag is None else BF16_LSE_ABS + LSE_ROUND_REL * lse_mag
        assert np.all(dl <= allow), f"{what}: max|dLSE|={dl.max():.3e}"
    return d.max()


def check_fp8(out, ref_out, what=""):
    """The FP8 gate: max |d out| <= 6e-2 (plus the bf16 output's half ulp,
    2^-8 |ref|) and mean <= 5e-3."""
    d = np.abs(out - ref_out)
    bound = FP8_OUT_MAX + BF16_OUT_REL_ROUND * np.abs(ref_out)
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    worst = np.unravel_index(np.argmax(d - bound), d.shape)
    print(f"{what}: max|dout|={d.max():.3e} mean={d.mean():.2e}", flush=True)
    assert np.all(d <= bound), f"{what}: max|dout|={d.max():.3e} at {worst} (ref {ref_out[worst]:.4f} got {out[worst]:.4f})"
    assert d.mean() <= FP8_OUT_MEAN, f"{what}: mean|dout|={d.mean():.3e}"
    return d.max(), d.mean()


def fp8_known_limit(out, ref_out, allowance, what=""):
    """The fast FP8 modes where they do not meet the max gate: on
    activation-like inputs (the FP8 matrix instructions' score sums; see
    FP8_MFMA_REL) and on rows with a handful of keys of nearly equal weight
    (the e4m3 rounding of the probabilities; see FP8_P_REL). Prints the
    literal max and the number of elements over the gate, holds the mean
    gate, and, as a separate diagnostic, checks that every element stays
    within the gate plus the error that the named cause explains (allowance:
    per row, leading axes of out). The precise mode meets the gate itself
    (check_fp8)."""
    d = np.abs(out - ref_out)
    bound = FP8_OUT_MAX + BF16_OUT_REL_ROUND * np.abs(ref_out)
    over = int(np.count_nonzero(d > bound))
    print(f"{what}: KNOWN LIMIT literal max|dout|={d.max():.3e}, {over} of {d.size} elements over the 6e-2 gate, "
          f"mean={d.mean():.2e}", flush=True)
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    assert d.mean() <= FP8_OUT_MEAN, f"{what}: mean|dout|={d.mean():.3e}"
    diag = bound + allowance[..., None]
    assert np.all(d <= diag), f"{what}: error beyond what FP8 score precision explains: max {d.max():.3e}"
    return d.max(), d.mean(), over


# An e4m3 value keeps 3 mantissa bits, so rounding a normal probability to
# nearest moves it by at most 2^-4 of itself; with the per-block scaling a
# probability below 2^-6 of its block's largest is subnormal and moves by at
# most 2^-10 of that largest one, at most 2^-10 of the row's largest weight
# (FP8_P_ABS allows twice that). On a row with two keys of weights w0, w1
# the output can move by up to w0 w1 2^-4 |v1 - v0|: over 6e-2 for
# |v1 - v0| ~ 4.
FP8_P_REL = 2.0 ** -4
FP8_P_ABS = 2.0 ** -9


FP8_P_BLOCK = 32   # keys per power-of-two scale block of the FP8 kernels (aligned at key 0)


def _p_rounding_terms(qh, kh, scale, i, nkeys, absc):
    """Exact weights w of row i over its visible keys 0..nkeys-1 and the
    absolute terms a_j = min(absc * (largest weight of j's scale block), w_j)."""
    s = (kh[:nkeys] @ qh[i]) * scale
    w = np.exp(s - s.max())
    w /= w.sum()
    starts = np.arange(0, nkeys, FP8_P_BLOCK)
    bmax = np.repeat(np.maximum.reduceat(w, starts), FP8_P_BLOCK)[:nkeys]
    return w, np.minimum(absc * bmax, w)


def _visible(rows, nkeys):
    rows = np.asarray(rows)
    return rows, (rows + 1 if nkeys is None else np.asarray(nkeys))


def fp8_p_rounding_allowance(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, rows,
                             rel: float = FP8_P_REL, absc: float = FP8_P_ABS, nkeys=None) -> np.ndarray:
    """Per-row bound on |d out| caused by rounding the probabilities to e4m3
    alone (a diagnostic of that known limit, never part of the gate).

    With the exact softmax weights w_j of row i and o = sum_j w_j v_j, weights
    perturbed to w_j (1 + d_j) + a_j (|d_j| <= rel, and |a_j| <= min(absc
    b_j, w_j) with b_j the largest weight of key j's 32-key scale block: the
    kernels scale each block so that its largest probability lands in [1, 2),
    and a probability too small for a normal code there is rounded to a
    subnormal one or to zero, never by more than itself) give
    o' - o = sum_j (w_j d_j + a_j) (v_j - o) / sum_j (w_j (1 + d_j) + a_j),
    since sum_j w_j (v_j - o) = 0. Returns, per row, the maximum over the
    columns of that bound (infinite where rel + sum_j a_j reaches 1). rel =
    2^-4 is rounding to nearest; 2^-3 (one code step) also covers a code that
    the kernel's fp32 score rounds the other way at a tie, and lean P, whose
    value 2^floor(y) (1 + frac(y)) stays within about 9 % of 2^y; lean P
    writes code 0 for probabilities below 2^-7 of their block's scale
    (absc = 2^-5 covers it; exact P's subnormals lie below 2^-6 of it and
    move by at most 2^-10 of it: absc = 2^-9). Row i sees keys 0..i, or
    0..nkeys[r]-1 when nkeys is given (range calls)."""
    rows, nk = _visible(rows, nkeys)
    out = np.empty(rows.shape[0])
    for r, i in enumerate(rows):
        n = int(nk[r])
        if n <= 0:
            out[r] = 0.0
            continue
        w, a = _p_rounding_terms(qh, kh, scale, i, n, absc)
        o = w @ vh[:n]
        dev = np.abs(vh[:n] - o)                           # (keys, d_v)
        num = rel * (w @ dev) + a @ dev
        den = 1.0 - rel - a.sum()
        out[r] = (num / den).max() if den > 0.0 else math.inf
    return out


def fp8_p_rounding_lse_allowance(qh: np.ndarray, kh: np.ndarray, scale: float, rows, rel: float = FP8_P_REL,
                                 absc: float = FP8_P_ABS, nkeys=None) -> np.ndarray:
    """Per-row bound on |d LSE| (natural log) from the same perturbed weights
    as fp8_p_rounding_allowance: the rounded sum lies within a factor
    (1 +- (rel + sum_j a_j)) of the exact one, so |d LSE| <= -ln(1 - rel -
    sum_j a_j) (infinite where rel + sum_j a_j reaches 1)."""
    rows, nk = _visible(rows, nkeys)
    out = np.empty(rows.shape[0])
    for r, i in enumerate(rows):
        n = int(nk[r])
        if n <= 0:
            out[r] = 0.0
            continue
        _, a = _p_rounding_terms(qh, kh, scale, i, n, absc)
        x = 1.0 - rel - a.sum()
        out[r] = -math.log(x) if x > 0.0 else math.inf
    return out


# gfx950's FP8 matrix instructions (v_mfma_scale_f32_16x16x128_f8f6f4 and the
# older v_mfma_f32_16x16x32_fp8_fp8) do not sum their products at fp32
# precision: measured on the GPU, the error of one 128-term FP8 dot product
# reaches 2^-11.5 of sum_c |a_c b_c| on activation-like operands (2^-15.7 on
# Gaussian ones), against 2^-22 for the bf16 instruction on the same values.
# Any kernel that computes q.k with them inherits this; on rows whose scores
# are huge (activation-like inputs: |s| ~ 2000 in log2 units) it moves the
# softmax weights of near-tied keys. FP8_MFMA_REL bounds it.
FP8_MFMA_REL = 2.0 ** -11


def fp8_score_allowance(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, rows) -> np.ndarray:
    """Per-row bound on |d out| caused by the FP8 MFMA's score error alone
    (a diagnostic of the known limit, never part of the gate).

    Each score carries an error of at most e_j = FP8_MFMA_REL * scale * log2(e)
    * sum_c |q_ic k_jc| (log2 units), so each softmax weight moves by at most a
    factor 2^(2 max_j e_j) and the weighted average of v by at most
    (2^(2 e_max) - 1) * max_j |v_j|."""
    rows = np.asarray(rows)
    nk = int(rows.max()) + 1
    mag = np.abs(qh[rows]) @ np.abs(kh[:nk]).T
    mag[np.arange(nk)[None, :] > rows[:, None]] = 0.0
    e = FP8_MFMA_REL * scale * np.log2(np.e) * mag.max(axis=1)
    vmax = np.abs(vh[:nk]).max()
    return (np.exp2(2 * e) - 1.0) * vmax


# Tight check against the model of this library's probability rounding
# (tests/fp8_rounding_model.py; a regression check, not the accuracy gate). What still differs is the score: the kernel's FP8
# MFMA sums in fp32 with its own rounding (bounded by 2^-15.7 sum|ab| on
# N(0, 1) data), so a code whose 8 y + C (lean) or 2^y (exact) lies that
# close to a rounding boundary can land one code step (at most 2^(1/8), 9%)
# away from the oracle's, and the lazy reference can move on the other side
# of its threshold. Single flips dominate the max; the mean stays tiny.
FP8_ROUND_MAX = 2e-2
FP8_ROUND_MEAN = 2e-4
FP8_ROUND_LSE_MAX = 1e-2
FP8_ROUND_LSE_MEAN = 1e-4


# One probability landing one code step away from the model's moves its
# weight w_j by at most 2^-3 w_j (a mantissa step of e4m3 is at most 2^-3 of
# the value; a lean code step 2^(1/8) - 1 < 2^-3), so, with weights summing
# to 1, the row's output by at most 2^-3 w_j max_c |v_jc - o_c| / (1 - 2^-3
# w_j) and its LSE by at most -ln(1 - 2^-3 w_j).
FP8_FLIP_REL = 2.0 ** -3
FP8_FLIP_ROWS = 2e-2        # rows with a flip, at most (at least 4 allowed)


def fp8_code_flip_bounds(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float, rows):
    """Per-row (out, LSE) bounds of one code flip of the worst key, from the
    exact softmax weights (a diagnostic allowance of check_fp8_rounding)."""
    rows = np.asarray(rows)
    ob = np.empty(rows.shape[0])
    lb = np.empty(rows.shape[0])
    for r, i in enumerate(rows):
        s = (kh[: i + 1] @ qh[i]) * scale
        w = np.exp(s - s.max())
        w /= w.sum()
        o = w @ vh[: i + 1]
        dev = np.abs(vh[: i + 1] - o).max(axis=1)
        step = FP8_FLIP_REL * w
        ob[r] = (step * dev / (1.0 - step)).max()
        lb[r] = -math.log(1.0 - step.max())
    return ob, lb


def check_fp8_rounding(out, ref_out, lse, ref_lse, what="", flip=None, flip_lse=None):
    """The kernel against the rounding model. flip, flip_lse (per row of
    out's leading axes, from fp8_code_flip_bounds): where given, an element
    may pass the tight bound by what one code flip in its row explains, in
    at most FP8_FLIP_ROWS of the rows (at least 4; a flip moves every
    column of its row), and the other rows keep the tight mean; the LSE of
    every row stays within the tight bound plus its flip bound, and the mean
    of all but the FP8_FLIP_ROWS largest LSE errors (at least 4) within the
    tight mean."""
    d = np.abs(out - ref_out)
    bound = FP8_ROUND_MAX + BF16_OUT_REL_ROUND * np.abs(ref_out)
    worst = np.unravel_index(np.argmax(d - bound), d.shape)
    over = int(np.count_nonzero(d > bound))
    stats = f"{what}: max|dout|={d.max():.3e} mean={d.mean():.3e} over the tight bound {over}"
    if lse is not None:
        dl = np.abs(lse - ref_lse)
        stats += f" max|dLSE|={dl.max():.3e} mean={dl.mean():.3e}"
    print(stats, flush=True)
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    if flip is None:
        assert np.all(d <= bound), f"{stats} worst at {worst} (ref {ref_out[worst]:.4f} got {out[worst]:.4f})"
        assert d.mean() <= FP8_ROUND_MEAN, stats
    else:
        # a flip moves every column of its row, so rows are counted; the
        # mean is taken over the rows without one
        flipped = (d > bound).reshape(d.shape[0], -1).any(axis=1)
        rows_over = int(np.count_nonzero(flipped))
        assert rows_over <= max(4, FP8_FLIP_ROWS * d.shape[0]), f"{stats}, in {rows_over} rows"
        assert np.all(d <= bound + flip[..., None]), f"{stats}: beyond one code flip at {worst}"
        rest = d[~flipped]
        assert rest.size == 0 or rest.mean() <= FP8_ROUND_MEAN, f"{stats} (mean of the other rows {rest.mean():.3e})"
    if lse is not None:
        assert np.all(np.isfinite(lse)), what + ": non-finite lse"
        if flip_lse is None:
            assert dl.max() <= FP8_ROUND_LSE_MAX and dl.mean() <= FP8_ROUND_LSE_MEAN, stats
        else:
            # rows with a flipped code are held to the flip bound; the mean
            # of the others (all but the FP8_FLIP_ROWS largest, at least 4)
            # stays tight
            assert np.all(dl <= FP8_ROUND_LSE_MAX + flip_lse), stats
            k = max(4, int(np.ceil(FP8_FLIP_ROWS * dl.size)))
            rest = np.sort(dl.ravel())[:-k]
            assert rest.size == 0 or rest.mean() <= FP8_ROUND_LSE_MEAN, f"{stats} (mean of the rest {rest.mean():.3e})"


def check_partial(out, ref_out, lse, ref_lse, what="", fp8=False):
    """Partial results over a key range: rows that see no key (oracle LSE
    -inf) must come back as out = 0 exactly and LSE = -inf; the others are
    held to the BF16 (or FP8) gate. out: (..., d) with lse shaped like its
    leading axes."""
    empty = np.isneginf(ref_lse)
    if lse is not None:
        assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf LSE rows differ"
    assert np.all(out[empty] == 0.0), f"{what}: rows that see no key are not zero"
    live = ~empty
    if not live.any():
        return
    if fp8:
        check_fp8(out[live], ref_out[live], what)
        if lse is not None:
            # the FP8 LSE comes from the rounded probabilities: one e4m3
            # rounding moves a row sum by at most 2^-4 relative, < 0.065 nats
            dl = np.abs(lse[live] - ref_lse[live])
            assert np.all(np.isfinite(dl)) and dl.max() < FP8_LSE_MAX, f"{what}: max|dLSE|={dl.max():.3e}"
    else:
        check_bf16(out[live], ref_out[live], None if lse is None else lse[live], None if lse is None else ref_lse[live],
                   what)


class tile_height:
    """Within the block, calls of one shape use query tiles of `tile_q` rows
    (128 or 256) instead of the library's automatic choice."""

    def __init__(self, zy, batch, seqlen, nheads, nheads_k, d_qk, dtype, tile_q):
        self.zy, self.shape, self.tile_q = zy, (batch, seqlen, nheads, nheads_k, d_qk, dtype), tile_q

    def __enter__(self):
        self.zy.zyfa_set_tile_q(*self.shape, tile_q=self.tile_q)
        return self

    def __exit__(self, *exc):
        self.zy.zyfa_set_tile_q(*self.shape, tile_q=0)
        return False
