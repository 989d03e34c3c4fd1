"""Pins of the float64 causal attention oracle (CPU only).

Each test checks the oracle against something other than itself: a closed
form, an invariant of the definition, brute force, or an independent
streaming formulation, chosen so that a dropped scale, a flipped mask, an
off-by-one on the diagonal, a wrong GQA mapping or a transposed operand
fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

from oracle import causal_attention_ref, causal_attention_rows_ref, causal_probs_ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(rng, B, S, H, Hk, dqk, dv, layout="bshd", std=1.0):
    def t(h, d):
        shp = (B, S, h, d) if layout == "bshd" else (B, h, S, d)
        return rng.standard_normal(shp) * std
    return t(H, dqk), t(Hk, dqk), t(Hk, dv)


def heads_view(x, layout):
    return np.swapaxes(x, 1, 2) if layout == "bshd" else x


def test_probability_rows_sum_to_one_and_are_causal():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal((37, 16)), rng.standard_normal((37, 16))
    p = causal_probs_ref(q, k, 0.25)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert np.all(p[np.triu_indices(37, 1)] == 0.0)
    assert np.all(p[np.tril_indices(37)] > 0.0)


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_row0_copies_v0_and_lse0_is_one_score(layout):
    rng = np.random.default_rng(1)
    B, S, H, Hk, dqk, dv = 2, 9, 4, 2, 24, 8
    q, k, v = rand_qkv(rng, B, S, H, Hk, dqk, dv, layout)
    scale = 0.3
    out, lse = causal_attention_ref(q, k, v, layout=layout, softmax_scale=scale)
    Q, K, V, O = (heads_view(x, layout) for x in (q, k, v, out))
    for b in range(B):
        for h in range(H):
            hk = h // (H // Hk)
            assert np.array_equal(O[b, h, 0], V[b, hk, 0])
            assert lse[b, h, 0] == pytest.approx(scale * Q[b, h, 0] @ K[b, hk, 0], abs=1e-12)


def test_constant_keys_give_causal_prefix_mean():
    rng = np.random.default_rng(2)
    B, S, H, d = 1, 50, 2, 16
    q = rng.standard_normal((B, S, H, d))
    kvec = rng.standard_normal(d)
    k = np.broadcast_to(kvec, (B, S, H, d)).copy()
    v = rng.standard_normal((B, S, H, d))
    scale = 1 / math.sqrt(d)
    out, lse = causal_attention_ref(q, k, v, softmax_scale=scale)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.allclose(out, prefix_mean, atol=1e-12, rtol=0)
    want_lse = scale * np.einsum("bshd,d->bhs", q, kvec) + np.log(np.arange(1, S + 1))[None, None, :]
    assert np.allclose(lse, want_lse, atol=1e-12, rtol=0)


def test_zero_queries_give_causal_prefix_mean():
    rng = np.random.default_rng(3)
    B, S, H, d = 1, 33, 1, 8
    q = np.zeros((B, S, H, d))
    k, v = rng.standard_normal((B, S, H, d)), rng.standard_normal((B, S, H, d))
    out, lse = causal_attention_ref(q, k, v)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    assert np.allclose(out, prefix_mean, atol=1e-12, rtol=0)
    assert np.allclose(lse[0, 0], np.log(np.arange(1, S + 1)), atol=1e-12, rtol=0)


def test_key_shift_invariance():
    # adding the same vector c to every key leaves O unchanged and shifts
    # LSE_i by scale * <q_i, c> (the K-smoothing argument of the README's
    # "Using FP8 attention in a model" section)
    rng = np.random.default_rng(4)
    B, S, H, d = 1, 40, 2, 16
    q, k, v = rand_qkv(rng, B, S, H, H, d, d)
    c = rng.standard_normal(d) * 3
    scale = 0.2
    o1, l1 = causal_attention_ref(q, k, v, softmax_scale=scale)
    o2, l2 = causal_attention_ref(q, k + c, v, softmax_scale=scale)
    assert np.allclose(o1, o2, atol=1e-12, rtol=0)
    assert np.allclose(l2 - l1, scale * np.einsum("bshd,d->bhs", q, c), atol=1e-11, rtol=0)


def _head_map_rows():
    with open(os.path.join(GOLD, "gqa_head_map.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            vals = [int(x) for x in line.split()]
            yield vals[0], vals[1], vals[2:]


@pytest.mark.parametrize("H,Hk,kvmap", list(_head_map_rows()))
def test_gqa_head_mapping_matches_golden(H, Hk, kvmap):
    # v of KV head j is constant j + 1: every output of query head h equals
    # its KV head's constant
    rng = np.random.default_rng(5)
    B, S, d = 1, 12, 8
    q = rng.standard_normal((B, S, H, d))
    k = rng.standard_normal((B, S, Hk, d))
    v = np.empty((B, S, Hk, d))
    for j in range(Hk):
        v[:, :, j, :] = j + 1
    out, _ = causal_attention_ref(q, k, v)
    for h in range(H):
        assert np.allclose(out[:, :, h, :], kvmap[h] + 1, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(6)
    B, S, H, Hk, d = 2, 20, 6, 2, 16
    q, k, v = rand_qkv(rng, B, S, H, Hk, d, d)
    o1, l1 = causal_attention_ref(q, k, v)
    o2, l2 = causal_attention_ref(q, np.repeat(k, H // Hk, axis=2), np.repeat(v, H // Hk, axis=2))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_layouts_agree():
    rng = np.random.default_rng(7)
    q, k, v = rand_qkv(rng, 2, 17, 4, 2, 24, 8, "bshd")
    o1, l1 = causal_attention_ref(q, k, v, layout="bshd")
    o2, l2 = causal_attention_ref(*(np.swapaxes(x, 1, 2) for x in (q, k, v)), layout="bhsd")
    assert np.allclose(np.swapaxes(o2, 1, 2), o1, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


@pytest.mark.parametrize("S,pad_to", [(1, 256), (63, 64), (100, 256), (257, 512)])
def test_zero_padding_is_exact_for_causal(S, pad_to):
    # "ZYFA" README, Usage: zero padding to a multiple of the tile gives the
    # exact result for causal attention, since no real query sees a padded key
    rng = np.random.default_rng(8)
    q, k, v = rand_qkv(rng, 1, S, 2, 1, 16, 8)
    o1, l1 = causal_attention_ref(q, k, v)
    padw = ((0, 0), (0, pad_to - S), (0, 0), (0, 0))
    o2, l2 = causal_attention_ref(np.pad(q, padw), np.pad(k, padw), np.pad(v, padw))
    # equal up to the summation order of the library matmul over a longer axis
    assert np.allclose(o2[:, :S], o1, atol=1e-13, rtol=0) and np.allclose(l2[:, :, :S], l1, atol=1e-13, rtol=0)


def _brute(qh, kh, vh, scale):
    """Scalar loops with math.fsum, one query at a time."""
    S, dv = qh.shape[0], vh.shape[1]
    out = np.zeros((S, dv))
    lse = np.zeros(S)
    for i in range(S):
        sc = [scale * math.fsum(qh[i, c] * kh[j, c] for c in range(qh.shape[1])) for j in range(i + 1)]
        m = max(sc)
        w = [math.exp(s - m) for s in sc]
        tot = math.fsum(w)
        for c in range(dv):
            out[i, c] = math.fsum(w[j] * vh[j, c] for j in range(i + 1)) / tot
        lse[i] = m + math.log(tot)
    return out, lse


def test_brute_force_tiny():
    rng = np.random.default_rng(9)
    B, S, H, Hk, dqk, dv = 1, 13, 3, 1, 7, 5
    q, k, v = rand_qkv(rng, B, S, H, Hk, dqk, dv, std=2.0)
    scale = 0.37
    out, lse = causal_attention_ref(q, k, v, softmax_scale=scale)
    for h in range(H):
        o, l = _brute(q[0, :, h], k[0, :, 0], v[0, :, 0], scale)
        assert np.allclose(out[0, :, h], o, atol=1e-12, rtol=0)
        assert np.allclose(lse[0, h], l, atol=1e-12, rtol=0)


def _online(qh, kh, vh, scale, block, tau):
    """Streaming softmax over key blocks with a lazy reference max: the
    reference moves only when a block's max passes it by more than tau."""
    S = qh.shape[0]
    out = np.zeros((S, vh.shape[1]))
    lse = np.zeros(S)
    for i in range(S):
        mref, l, acc = -np.inf, 0.0, np.zeros(vh.shape[1])
        for j0 in range(0, i + 1, block):
            j1 = min(i + 1, j0 + block)
            s = scale * (kh[j0:j1] @ qh[i])
            bm = s.max()
            if bm > mref + tau:
                new = bm
                if np.isfinite(mref):
                    f = math.exp(mref - new)
                    l *= f
                    acc *= f
                mref = new
            p = np.exp(s - mref)
            l += p.sum()
            acc += p @ vh[j0:j1]
        out[i] = acc / l
        lse[i] = mref + math.log(l)
    return out, lse


@pytest.mark.parametrize("block", [1, 3, 7, 64])
@pytest.mark.parametrize("tau", [0.0, 0.125 * math.log(2), 8 * math.log(2)])
def test_online_softmax_matches(block, tau):
    rng = np.random.default_rng(10)
    S, d = 150, 16
    q, k, v = rand_qkv(rng, 1, S, 1, 1, d, d, std=1.5)
    out, lse = causal_attention_ref(q, k, v)
    o, l = _online(q[0, :, 0], k[0, :, 0], v[0, :, 0], 1 / math.sqrt(d), block, tau)
    assert np.allclose(out[0, :, 0], o, atol=1e-12, rtol=0)
    assert np.allclose(lse[0, 0], l, atol=1e-12, rtol=0)


def test_lse_merge_over_key_ranges():
    # results over disjoint key ranges merge exactly through their LSE
    # ("ZYFA" README, Accuracy: the LSE lets results over different key
    # ranges be merged)
    rng = np.random.default_rng(11)
    S, d, t = 60, 8, 23
    qh, kh, vh = (rng.standard_normal((S, d)) for _ in range(3))
    scale = 0.5
    out, lse = causal_attention_ref(qh[None, :, None], kh[None, :, None], vh[None, :, None], softmax_scale=scale)
    for i in range(t, S):
        sc = scale * (kh[: i + 1] @ qh[i])
        a, b = sc[:t], sc[t:]
        la, lb = np.logaddexp.reduce(a), np.logaddexp.reduce(b)
        oa = np.exp(a - la) @ vh[:t]
        ob = np.exp(b - lb) @ vh[t: i + 1]
        l = np.logaddexp(la, lb)
        o = np.exp(la - l) * oa + np.exp(lb - l) * ob
        assert np.allclose(out[0, i, 0], o, atol=1e-12) and lse[0, 0, i] == pytest.approx(l, abs=1e-12)


def test_rows_helper_matches_full():
    rng = np.random.default_rng(12)
    for layout in ("bshd", "bhsd"):
        q, k, v = rand_qkv(rng, 2, 70, 4, 2, 24, 8, layout)
        out, lse = causal_attention_ref(q, k, v, layout=layout)
        O = heads_view(out, layout)
        rows = [0, 5, 31, 69]
        o, l = causal_attention_rows_ref(q, k, v, 1, 3, rows, layout=layout)
        assert np.allclose(o, O[1, 3, rows], atol=1e-13) and np.allclose(l, lse[1, 3, rows], atol=1e-13)


def test_default_scale_is_inverse_sqrt_dqk():
    rng = np.random.default_rng(13)
    q, k, v = rand_qkv(rng, 1, 10, 1, 1, 192, 128)
    o1 = causal_attention_ref(q, k, v, return_lse=False)
    o2 = causal_attention_ref(q, k, v, softmax_scale=1 / math.sqrt(192), return_lse=False)
    assert np.array_equal(o1, o2)
