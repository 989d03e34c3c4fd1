"""Seeded synthetic inputs for causal prefill attention.

This module is shared by the oracle-side tests and the GPU-side tests and
benchmark. It only draws random numbers and arranges them into the shapes of
the five workloads; it holds none of the attention arithmetic, none of the
rounding rules and none of the FP8 quantization rules. Values come out as
float32 numpy arrays; each side casts them to bf16 with its own code.

Workloads (all causal, seqlen_q == seqlen_k):

1. MHA bf16, batch 1, seqlen 256, 4 query / 4 KV heads, d_qk = d_v = 128,
   bshd, LSE requested.
2. GQA bf16, batch 1, seqlen 8192, 32 / 8 heads, d = 128, bshd, LSE.
3. GQA fp8 e4m3, batch 1, seqlen 16384, 32 / 8 heads, d = 128, bshd.
4. The per-head form of multi-head latent attention used in prefill:
   batch 1, seqlen 16384, 16 / 16 heads, d_qk = 192, d_v = 128, bhsd;
   bf16 and fp8.
5. GQA bf16 and fp8, batch 2, seqlen 32000, 32 / 8 heads, d = 128, bshd,
   with activation-like q and k (see ``activation_like``).

Recipe: ``numpy.random.Generator(PCG64(seed))`` with the seed equal to the
workload number; q, k and v are drawn in that order as float32 N(0, 1) of
the caller's layout. Workload 5 then draws, from the same generator, the
outlier channels and per-token log-scales described in ``activation_like``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    nheads_k: int
    d_qk: int
    d_v: int
    layout: str          # "bshd" or "bhsd"
    dtypes: tuple        # subset of ("bf16", "fp8")
    with_lse: bool
    activation_like: bool
    seed: int

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_qk))

    def flops(self) -> float:
        """Causal attention FLOPs as the ZYFA README counts them
        (Performance, kernel-benchmark protocol): B*H*S^2*(d_qk + d_v)."""
        return float(self.batch) * self.nheads * float(self.seqlen) ** 2 * (self.d_qk + self.d_v)

    def shape(self, which: str):
        d = self.d_v if which == "v" else self.d_qk
        h = self.nheads if which == "q" else self.nheads_k
        if self.layout == "bshd":
            return (self.batch, self.seqlen, h, d)
        return (self.batch, h, self.seqlen, d)

    def resized(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload("mha_bf16_s256", 1, 256, 4, 4, 128, 128, "bshd", ("bf16",), True, False, 1),
    2: Workload("gqa_bf16_s8192", 1, 8192, 32, 8, 128, 128, "bshd", ("bf16",), True, False, 2),
    3: Workload("gqa_fp8_s16384", 1, 16384, 32, 8, 128, 128, "bshd", ("fp8",), False, False, 3),
    4: Workload("mla_d192_s16384", 1, 16384, 16, 16, 192, 128, "bhsd", ("bf16", "fp8"), False, False, 4),
    5: Workload("gqa_act_s32000_b2", 2, 32000, 32, 8, 128, 128, "bshd", ("bf16", "fp8"), False, True, 5),
}


def _head_axis(layout: str) -> int:
    return 2 if layout == "bshd" else 1


def _seq_axis(layout: str) -> int:
    return 1 if layout == "bshd" else 2


def activation_like(rng: np.random.Generator, w: Workload, q: np.ndarray, k: np.ndarray) -> None:
    """In-place transform that makes q and k peaked like captured activations.

    Per KV head, four distinct channels are drawn; those channels are
    multiplied by 20 in that KV head of k and in every query head of its
    group (groups are consecutive query heads). Then one lognormal(0, 0.5)
    factor per token (b, s) multiplies all heads and channels of q, and an
    independently drawn one multiplies k. v is left N(0, 1).
    """
    ha, sa = _head_axis(w.layout), _seq_axis(w.layout)
    g = w.nheads // w.nheads_k
    for hk in range(w.nheads_k):
        ch = rng.choice(w.d_qk, size=4, replace=False)
        ks = [slice(None)] * 4
        ks[ha] = hk
        kview = k[tuple(ks)]
        kview[..., ch] *= np.float32(20.0)
        for h in range(hk * g, (hk + 1) * g):
            qs = [slice(None)] * 4
            qs[ha] = h
            qview = q[tuple(qs)]
            qview[..., ch] *= np.float32(20.0)
    for x in (q, k):
        fac = rng.lognormal(0.0, 0.5, size=(w.batch, w.seqlen)).astype(np.float32)
        if sa == 1:
            x *= fac[:, :, None, None]
        else:
            x *= fac[:, None, :, None]


def generate(w: Workload, seed: Optional[int] = None):
    """Draw (q, k, v) as float32 arrays in the workload's layout."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    q = rng.standard_normal(w.shape("q"), dtype=np.float32)
    k = rng.standard_normal(w.shape("k"), dtype=np.float32)
    v = rng.standard_normal(w.shape("v"), dtype=np.float32)
    if w.activation_like:
        activation_like(rng, w, q, k)
    return q, k, v


def sampled_heads(seed: int, seqlen: int, heads, d_qk: int, d_v: int):
    """Draw (q, k, v) for a few heads of a tensor too large to fill on the
    host: float32 N(0, 1) arrays of shape (len(heads), seqlen, d) each, in
    head order, q then k then v per head. The other heads of such a tensor
    are left zero by the caller."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = [[], [], []]
    for _ in heads:
        for i, d in enumerate((d_qk, d_qk, d_v)):
            out[i].append(rng.standard_normal((seqlen, d), dtype=np.float32))
    return tuple(np.stack(x) for x in out)
