"""Pins of the range-attention and LSE-merge oracle (oracle/partial.py)
against brute force, library routines and the whole-sequence oracle."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle


def _brute(q, k, v, q_pos0, k_pos0, scale):
    """Scalar loops with math.fsum: one (Sq, d) head, bshd-free."""
    Sq, Sk = q.shape[0], k.shape[0]
    out = np.zeros((Sq, v.shape[1]))
    lse = np.full(Sq, -math.inf)
    for i in range(Sq):
        vis = [j for j in range(Sk) if k_pos0 + j <= q_pos0 + i]
        if not vis:
            continue
        s = {j: scale * math.fsum(float(q[i, c]) * float(k[j, c]) for c in range(q.shape[1])) for j in vis}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in vis}
        tot = math.fsum(w.values())
        lse[i] = m + math.log(tot)
        for c in range(v.shape[1]):
            out[i, c] = math.fsum(w[j] * float(v[j, c]) for j in vis) / tot
    return out, lse


@pytest.mark.parametrize("Sq,Sk,q_pos0,k_pos0", [
    (5, 7, 2, 0),      # chunk of queries after a prefix
    (6, 4, 0, 3),      # negative offset: rows 0..2 see nothing
    (4, 6, 10, 0),     # every key visible
    (3, 5, 0, 9),      # nothing visible
    (7, 7, 0, 0),      # plain causal
])
def test_range_matches_brute_force(Sq, Sk, q_pos0, k_pos0):
    rng = np.random.default_rng(Sq * 100 + Sk)
    q, k, v = rng.standard_normal((Sq, 6)), rng.standard_normal((Sk, 6)), rng.standard_normal((Sk, 5))
    o, l = oracle.range_attention_ref(q[None, :, None], k[None, :, None], v[None, :, None], q_pos0, k_pos0,
                                      softmax_scale=0.7)
    bo, bl = _brute(q, k, v, q_pos0, k_pos0, 0.7)
    np.testing.assert_allclose(o[0, :, 0], bo, atol=1e-13)
    assert np.array_equal(np.isinf(l[0, 0]), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(l[0, 0][fin], bl[fin], atol=1e-12)


def test_no_visible_key_gives_zero_and_minus_inf():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((1, 8, 2, 16)), rng.standard_normal((1, 8, 1, 16)), rng.standard_normal((1, 8, 1, 16))
    o, l = oracle.range_attention_ref(q, k, v, 0, 5)
    assert np.all(o[0, :5] == 0.0) and np.all(np.isneginf(l[0, :, :5]))
    assert np.all(np.isfinite(l[0, :, 5:]))


def test_all_visible_is_plain_softmax_attention():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((9, 32)), rng.standard_normal((11, 32)), rng.standard_normal((11, 8))
    o, l = oracle.range_attention_ref(q[None, :, None], k[None, :, None], v[None, :, None], 100, 0)
    sc = (q @ k.T) / np.sqrt(32)
    np.testing.assert_allclose(o[0, :, 0], softmax(sc, axis=1) @ v, atol=1e-13)
    np.testing.assert_allclose(l[0, 0], logsumexp(sc, axis=1), atol=1e-13)


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_chunk_equals_last_rows_of_whole_sequence(layout):
    rng = np.random.default_rng(5)
    S, Sq = 40, 13
    shp = lambda s, h, d: (1, s, h, d) if layout == "bshd" else (1, h, s, d)
    q = rng.standard_normal(shp(S, 4, 16))
    k, v = rng.standard_normal(shp(S, 2, 16)), rng.standard_normal(shp(S, 2, 16))
    fo, fl = oracle.causal_attention_ref(q, k, v, layout=layout)
    qc = q[:, S - Sq:] if layout == "bshd" else q[:, :, S - Sq:]
    o, l = oracle.range_attention_ref(qc, k, v, S - Sq, 0, layout=layout)
    want = fo[:, S - Sq:] if layout == "bshd" else fo[:, :, S - Sq:]
    np.testing.assert_allclose(o, want, atol=1e-13)
    np.testing.assert_allclose(l, fl[:, :, S - Sq:], atol=1e-13)


def test_whole_range_equals_causal_oracle():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((2, 30, 4, 8)), rng.standard_normal((2, 30, 1, 8)), rng.standard_normal((2, 30, 1, 8))
    fo, fl = oracle.causal_attention_ref(q, k, v)
    o, l = oracle.range_attention_ref(q, k, v, 7, 7)
    np.testing.assert_allclose(o, fo, atol=1e-13)
    np.testing.assert_allclose(l, fl, atol=1e-13)


@pytest.mark.parametrize("split", [0, 1, 17, 29, 30])
def test_merge_of_key_splits_is_the_whole(split):
    rng = np.random.default_rng(7)
    S = 30
    q, k, v = rng.standard_normal((1, S, 2, 8)), rng.standard_normal((1, S, 2, 8)), rng.standard_normal((1, S, 2, 8))
    fo, fl = oracle.causal_attention_ref(q, k, v)
    oa, la = oracle.range_attention_ref(q, k[:, :split], v[:, :split], 0, 0)
    ob, lb = oracle.range_attention_ref(q, k[:, split:], v[:, split:], 0, split)
    o, l = oracle.lse_merge_layout_ref(oa, la, ob, lb, "bshd")
    np.testing.assert_allclose(o, fo, atol=1e-13)
    np.testing.assert_allclose(l, fl, atol=1e-13)


def test_merge_identities():
    rng = np.random.default_rng(8)
    oa, ob, oc = (rng.standard_normal((5, 4)) for _ in range(3))
    la, lb, lc = (rng.standard_normal(5) * 3 for _ in range(3))
    # an empty partial leaves the other unchanged
    o, l = oracle.lse_merge_ref(oa, la, ob, np.full(5, -np.inf))
    assert np.array_equal(o, oa) and np.array_equal(l, la)
    # both empty: zero output, -inf
    o, l = oracle.lse_merge_ref(oa, np.full(5, -np.inf), ob, np.full(5, -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # commutative and associative
    o1, l1 = oracle.lse_merge_ref(oa, la, ob, lb)
    o2, l2 = oracle.lse_merge_ref(ob, lb, oa, la)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    o3, l3 = oracle.lse_merge_ref(*oracle.lse_merge_ref(oa, la, ob, lb), oc, lc)
    o4, l4 = oracle.lse_merge_ref(oa, la, *oracle.lse_merge_ref(ob, lb, oc, lc))
    np.testing.assert_allclose(o3, o4, atol=1e-13)
    np.testing.assert_allclose(l3, l4, atol=1e-13)
    # the weights: closed form for equal LSEs is the mean and LSE + ln 2
    o, l = oracle.lse_merge_ref(oa, la, ob, la)
    np.testing.assert_allclose(o, (oa + ob) / 2, atol=1e-15)
    np.testing.assert_allclose(l, la + np.log(2), atol=1e-14)
