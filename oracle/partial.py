"""Attention over a range of key positions, and the LSE merge of partial
results, in float64 (oracle; test infrastructure only).

What is computed, from the pages:
- "ZYFA" README, Accuracy: the log-sum-exp comes back with the output so
  that outputs over disjoint key ranges can be combined into the whole.
- flash-attention RDNA3 extension page, kernel notes: a split of the keys
  across workers yields partial outputs with their LSE, combined by an LSE
  reduction.

Positions: query row i of the call sits at position q_pos0 + i and key j
at k_pos0 + j; key j is visible to row i when k_pos0 + j <= q_pos0 + i (the
causal rule on absolute positions). With H, Hk and h_k = floor(h Hk / H)
as for whole-sequence attention:

    Sc[i, j] = scale * <Q[i], K[j]>   if visible, else -inf
    LSE_i    = ln sum_j exp(Sc[i, j])            (-inf when nothing is visible)
    O[i]     = sum_j exp(Sc[i, j] - LSE_i) V[j]  (0 when nothing is visible)

Merge of two results of the same query rows over disjoint key sets A, B:

    LSE = ln(exp(LSE_A) + exp(LSE_B))
    O   = exp(LSE_A - LSE) O_A + exp(LSE_B - LSE) O_B

which is the result over A and B together (0 and -inf when both are empty).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import _split, kv_head


def _range_head(qh, kh, vh, scale, rows, q_pos0, k_pos0):
    """O and LSE of the given rows of one head."""
    rows = np.asarray(rows, dtype=np.int64)
    if kh.shape[0] == 0:                # an empty key range
        return np.zeros((len(rows), vh.shape[1])), np.full(len(rows), -np.inf)
    sc = scale * (qh[rows] @ kh.T)
    kpos = k_pos0 + np.arange(kh.shape[0], dtype=np.int64)
    qpos = q_pos0 + rows
    sc[kpos[None, :] > qpos[:, None]] = -np.inf
    m = sc.max(axis=1, keepdims=True)
    seen = np.isfinite(m[:, 0])
    m[~seen] = 0.0                      # rows that see no key: exp(-inf) = 0
    p = np.exp(sc - m)
    l = p.sum(axis=1, keepdims=True)
    o = np.zeros((len(rows), vh.shape[1]))
    o[seen] = (p[seen] @ vh) / l[seen]
    lse = np.full(len(rows), -np.inf)
    lse[seen] = m[seen, 0] + np.log(l[seen, 0])
    return o, lse


def range_attention_ref(q, k, v, q_pos0: int, k_pos0: int, *, layout: str = "bshd",
                        softmax_scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """q: (B, Sq, H, d_qk) or (B, H, Sq, d_qk); k, v with Sk positions and Hk
    heads. Returns (out in q's layout with head dim d_v, LSE (B, H, Sq))."""
    Q, K, V = (_split(np.asarray(x, dtype=np.float64), layout) for x in (q, k, v))
    B, H, Sq, dqk = Q.shape
    Hk = K.shape[1]
    if H % Hk:
        raise ValueError("nheads must be a multiple of nheads_k")
    scale = (1.0 / np.sqrt(dqk)) if softmax_scale is None else float(softmax_scale)
    O = np.zeros((B, H, Sq, V.shape[3]))
    L = np.zeros((B, H, Sq))
    rows = np.arange(Sq)
    for b in range(B):
        for h in range(H):
            hk = kv_head(h, H, Hk)
            O[b, h], L[b, h] = _range_head(Q[b, h], K[b, hk], V[b, hk], scale, rows, q_pos0, k_pos0)
    return (np.swapaxes(O, 1, 2) if layout == "bshd" else O), L


def range_attention_rows_ref(q, k, v, b: int, h: int, rows, q_pos0: int, k_pos0: int, *,
                             layout: str = "bshd", softmax_scale: Optional[float] = None):
    """O (len(rows), d_v) and LSE of selected rows of one (batch, head)."""
    Q, K, V = (_split(np.asarray(x), layout) for x in (q, k, v))
    H, Hk, dqk = Q.shape[1], K.shape[1], Q.shape[3]
    scale = (1.0 / np.sqrt(dqk)) if softmax_scale is None else float(softmax_scale)
    hk = kv_head(h, H, Hk)
    return _range_head(Q[b, h].astype(np.float64), K[b, hk].astype(np.float64), V[b, hk].astype(np.float64),
                       scale, rows, q_pos0, k_pos0)


def lse_merge_ref(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Merge two partial results of the same rows. o_*: (..., d); lse_*:
    (...) matching o_*'s leading axes. Returns (O, LSE)."""
    o_a, o_b = np.asarray(o_a, dtype=np.float64), np.asarray(o_b, dtype=np.float64)
    la, lb = np.asarray(lse_a, dtype=np.float64), np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    empty = ~np.isfinite(m)
    ms = np.where(empty, 0.0, m)
    wa, wb = np.exp(la - ms), np.exp(lb - ms)
    tot = wa + wb
    lse = np.where(empty, -np.inf, ms + np.log(np.where(empty, 1.0, tot)))
    den = np.where(empty, 1.0, tot)
    o = (wa / den)[..., None] * o_a + (wb / den)[..., None] * o_b
    return o, lse


def lse_merge_layout_ref(o_a, lse_a, o_b, lse_b, layout: str = "bshd"):
    """lse_merge_ref for outputs in a (B, S, H, d) or (B, H, S, d) layout and
    LSE (B, H, S)."""
    A, Bo = _split(np.asarray(o_a), layout), _split(np.asarray(o_b), layout)
    o, lse = lse_merge_ref(A, lse_a, Bo, lse_b)
    return (np.swapaxes(o, 1, 2) if layout == "bshd" else o), lse
