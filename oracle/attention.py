"""Causal forward attention in float64 (oracle; test infrastructure only).

Definition, from the "ZYFA" README:
- Supported configurations: causal forward pass with seqlen_q == seqlen_k;
  nheads a multiple of nheads_k (MHA, GQA, MQA); d_qk = d_v = 128 or
  d_qk = 192 with d_v = 128; layouts (batch, seqlen, heads, head_dim) or
  (batch, heads, seqlen, head_dim).
- Usage: return_lse gives the log-sum-exp of each row of scaled scores,
  natural log, shape (batch, heads, seqlen).
- Accuracy: errors are measured against fp64 attention on the same
  (quantized) inputs; FP8 inputs enter as code value times descale.

For batch b and query head h, the KV head is h_k = floor(h * nheads_k /
nheads): consecutive query heads share a KV head, as in flash-attn's
grouped-query convention. With Q = q[b, :, h], K = k[b, :, h_k],
V = v[b, :, h_k] (rows are positions):

    Sc[i, j] = scale * <Q[i], K[j]>          for j <= i, and -inf for j > i
    m_i      = max_j Sc[i, j]
    l_i      = sum_j exp(Sc[i, j] - m_i)
    O[i]     = sum_j exp(Sc[i, j] - m_i) * V[j] / l_i
    LSE_i    = m_i + ln(l_i)

The score matrix is materialised in blocks of query rows against all keys
(the mask is applied by setting entries to -inf), with no online softmax,
no tiling of the key axis and no reordering beyond numpy's own matmul.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

ROW_BLOCK = 2048


def _split(x: np.ndarray, layout: str) -> np.ndarray:
    """Return a (batch, heads, seqlen, d) view of x."""
    if layout == "bshd":
        return np.swapaxes(x, 1, 2)
    if layout == "bhsd":
        return x
    raise ValueError(f"unknown layout {layout!r}")


def kv_head(h: int, nheads: int, nheads_k: int) -> int:
    return (h * nheads_k) // nheads


def causal_probs_ref(qh: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """Full S x S causal softmax matrix of one head (rows are queries)."""
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    s = qh.shape[0]
    sc = scale * (qh @ kh.T)
    mask = np.triu(np.ones((s, s), dtype=bool), k=1)
    sc[mask] = -np.inf
    m = sc.max(axis=1, keepdims=True)
    p = np.exp(sc - m)
    return p / p.sum(axis=1, keepdims=True)


def _head_rows(qh, kh, vh, scale, rows):
    """O and LSE for the given query rows of one head."""
    rows = np.asarray(rows, dtype=np.int64)
    sc = scale * (qh[rows] @ kh.T)                       # (r, S)
    keys = np.arange(kh.shape[0], dtype=np.int64)
    sc[keys[None, :] > rows[:, None]] = -np.inf
    m = sc.max(axis=1, keepdims=True)
    p = np.exp(sc - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vh) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def causal_attention_ref(q, k, v, *, layout: str = "bshd",
                         softmax_scale: Optional[float] = None,
                         heads: Optional[Iterable[int]] = None,
                         return_lse: bool = True):
    """Causal attention of whole tensors.

    q: (B, S, H, d_qk) or (B, H, S, d_qk); k likewise with nheads_k heads;
    v with d_v. Values are converted to float64. Returns (out, lse) with out
    in q's layout and head dim d_v (float64), lse (B, H, S) float64.
    ``heads`` restricts the computation to some query heads (others are NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Q, K, V = _split(q, layout), _split(k, layout), _split(v, layout)
    B, H, S, dqk = Q.shape
    Hk = K.shape[1]
    if H % Hk:
        raise ValueError("nheads must be a multiple of nheads_k")
    scale = (1.0 / np.sqrt(dqk)) if softmax_scale is None else float(softmax_scale)
    dv = V.shape[3]
    O = np.full((B, H, S, dv), np.nan)
    L = np.full((B, H, S), np.nan)
    hs = range(H) if heads is None else heads
    for b in range(B):
        for h in hs:
            hk = kv_head(h, H, Hk)
            for r0 in range(0, S, ROW_BLOCK):
                rows = np.arange(r0, min(S, r0 + ROW_BLOCK))
                o, lse = _head_rows(Q[b, h], K[b, hk], V[b, hk], scale, rows)
                O[b, h, rows] = o
                L[b, h, rows] = lse
    out = np.swapaxes(O, 1, 2) if layout == "bshd" else O
    return (out, L) if return_lse else out


def causal_attention_rows_ref(q, k, v, b: int, h: int, rows, *, layout: str = "bshd",
                              softmax_scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O (len(rows), d_v) and LSE (len(rows),) of selected query rows of one
    (batch, head), for spot checks at sizes too large to compute whole."""
    Q, K, V = _split(np.asarray(q), layout), _split(np.asarray(k), layout), _split(np.asarray(v), layout)
    H, Hk = Q.shape[1], K.shape[1]
    dqk = Q.shape[3]
    scale = (1.0 / np.sqrt(dqk)) if softmax_scale is None else float(softmax_scale)
    hk = kv_head(h, H, Hk)
    rows = np.asarray(rows, dtype=np.int64)
    nkeys = int(rows.max()) + 1          # keys past the last row are masked for every row
    qh = Q[b, h].astype(np.float64)
    kh = K[b, hk, :nkeys].astype(np.float64)
    vh = V[b, hk, :nkeys].astype(np.float64)
    return _head_rows(qh, kh, vh, scale, rows)
