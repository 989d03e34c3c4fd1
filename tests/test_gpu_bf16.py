"""GPU parity of the BF16 path against the float64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, Workload, generate
from parity import bf16_pair, check_bf16, out_to_f64, score_magnitude, tile_height

pytestmark = pytest.mark.gpu

zy = pytest.importorskip("causal_flashattention_prefill_amd")


def run_case(w: Workload, seed=None, with_lse=True, heads=None):
    q, k, v = generate(w, seed)
    (tq, rq), (tk, rk), (tv, rv) = bf16_pair(q), bf16_pair(k), bf16_pair(v)
    print(f"case {w.name} B{w.batch} S{w.seqlen} H{w.nheads}/{w.nheads_k} d{w.d_qk}/{w.d_v} {w.layout}", flush=True)
    res = zy.zyfa_fwd(tq, tk, tv, layout=w.layout, return_lse=with_lse)
    torch.cuda.synchronize()
    out, lse = res if with_lse else (res, None)
    ref_out, ref_lse = oracle.causal_attention_ref(rq, rk, rv, layout=w.layout, heads=heads)
    o = out_to_f64(out)
    if heads is not None:
        hax = 2 if w.layout == "bshd" else 1
        o = np.take(o, heads, axis=hax)
        ref_out = np.take(ref_out, heads, axis=hax)
        ref_lse = ref_lse[:, heads]
    l = None if lse is None else lse.cpu().numpy().astype(np.float64)
    if l is not None and heads is not None:
        l = l[:, heads]
    mag = None
    if w.activation_like and with_lse:
        mag = _magnitudes(rq, rk, w, heads)
    return check_bf16(o, ref_out, l, ref_lse if with_lse else None, w.name, lse_mag=mag)


def _heads_view(x, layout):
    return np.swapaxes(x, 1, 2) if layout == "bshd" else x


def _magnitudes(rq, rk, w, heads=None):
    Q, K = _heads_view(rq, w.layout), _heads_view(rk, w.layout)
    hs = range(w.nheads) if heads is None else heads
    g = w.nheads // w.nheads_k
    rows = np.arange(w.seqlen)
    return np.stack([np.stack([score_magnitude(Q[b, h], K[b, h // g], w.softmax_scale, rows) for h in hs])
                     for b in range(w.batch)])


def test_workload1_full():
    run_case(WORKLOADS[1])


@pytest.mark.parametrize("with_lse", [True, False])
@pytest.mark.parametrize("B,S,H,Hk,dqk,layout", [
    (2, 700, 4, 2, 128, "bshd"),     # several tiles, ragged tail, GQA, 2 batches
    (1, 1000, 4, 1, 128, "bhsd"),    # MQA, bhsd, ragged
    (1, 600, 2, 2, 192, "bhsd"),     # d_qk = 192
    (2, 520, 3, 3, 192, "bshd"),
    (1, 1, 2, 1, 128, "bshd"),       # single token
    (1, 63, 2, 2, 128, "bshd"),
    (1, 255, 2, 2, 128, "bhsd"),
    (1, 257, 2, 1, 128, "bshd"),
    (1, 4097, 2, 1, 128, "bshd"),
    (37, 100, 6, 2, 128, "bshd"),    # many short sequences: one partial tile per slice
    (37, 100, 4, 4, 192, "bhsd"),
])
@pytest.mark.parametrize("tile_q", [256, 128])
def test_small_shapes(B, S, H, Hk, dqk, layout, with_lse, tile_q):
    w = Workload("small", B, S, H, Hk, dqk, 128, layout, ("bf16",), True, False, 1000 + S)
    print(f"tile_q {tile_q}", flush=True)
    with tile_height(zy, B, S, H, Hk, dqk, zy.DTYPE_BF16, tile_q):
        run_case(w, with_lse=with_lse)


@pytest.mark.parametrize("tile_q", [128, 256])
def test_several_rounds_of_jobs(tile_q):
    # 512 pair jobs of 128-row tiles (256 of 256-row tiles): the persistent
    # workgroups take two jobs each at the lower height
    B, S, H, Hk = 2, 4096, 16, 4
    w = Workload("rounds", B, S, H, Hk, 128, 128, "bshd", ("bf16",), True, False, 4242)
    print(f"tile_q {tile_q}", flush=True)
    with tile_height(zy, B, S, H, Hk, 128, zy.DTYPE_BF16, tile_q):
        run_case(w, with_lse=True, heads=[0, 5, 15])


def test_no_lse_variant_workload1():
    # without LSE the kernel divides by the matrix-unit sum of the rounded P
    run_case(WORKLOADS[1], with_lse=False)


def test_activation_like_small():
    w = WORKLOADS[5].resized(batch=1, seqlen=1536, name="act_small")
    run_case(w)


def _sample_rows(S, rng, n=24):
    base = [0, 1, 2, 63, 64, 65, 255, 256, 257, S // 2, S - 257, S - 256, S - 65, S - 2, S - 1]
    rows = set(r for r in base if 0 <= r < S)
    rows.update(rng.integers(0, S, n).tolist())
    return sorted(rows)


@pytest.mark.parametrize("with_lse", [True, False])
@pytest.mark.parametrize("wid", [2, 4, 5, "3share"])
def test_full_size_sampled_rows(wid, with_lse):
    # the benchmark's shapes; the oracle computes sampled rows one by one.
    # "3share": one GPU's share of the 16K GQA shape over 8 GPUs (4 / 1
    # heads), which runs on 128-row query tiles
    w = WORKLOADS[3].resized(nheads=4, nheads_k=1, name="gqa_s16384_share8") if wid == "3share" else WORKLOADS[wid]
    q, k, v = generate(w)
    (tq, rq), (tk, rk), (tv, rv) = bf16_pair(q), bf16_pair(k), bf16_pair(v)
    print(f"case full {w.name}", flush=True)
    res = zy.zyfa_fwd(tq, tk, tv, layout=w.layout, return_lse=with_lse)
    torch.cuda.synchronize()
    out, lse = res if with_lse else (res, None)
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64) if with_lse else None
    rng = np.random.default_rng(33 if wid == "3share" else wid)
    for b in range(w.batch):
        for h in sorted(set([0, w.nheads - 1] + rng.integers(0, w.nheads, 2).tolist())):
            rows = _sample_rows(w.seqlen, rng)
            ro, rl = oracle.causal_attention_rows_ref(rq, rk, rv, b, h, rows, layout=w.layout)
            got = o[b, rows, h] if w.layout == "bshd" else o[b, h, rows]
            mag = None
            if w.activation_like:
                Q, K = _heads_view(rq, w.layout), _heads_view(rk, w.layout)
                mag = score_magnitude(Q[b, h], K[b, h // (w.nheads // w.nheads_k)], w.softmax_scale, rows)
            check_bf16(got, ro, l[b, h, rows] if with_lse else None, rl if with_lse else None,
                       f"{w.name} b{b} h{h}", lse_mag=mag)


def test_bitwise_deterministic():
    w = WORKLOADS[2].resized(seqlen=2048)
    q, k, v = generate(w)
    tq, tk, tv = (bf16_pair(x)[0] for x in (q, k, v))
    plain = zy.zyfa_fwd(tq, tk, tv)
    for i in range(5):
        assert torch.equal(zy.zyfa_fwd(tq, tk, tv), plain), f"no-LSE run {i} differs"
    q, k, v = generate(w)
    tq, tk, tv = (bf16_pair(x)[0] for x in (q, k, v))
    first, flse = zy.zyfa_fwd(tq, tk, tv, return_lse=True)
    a = torch.randn(2048, 2048, device="cuda")
    for i in range(10):
        if i % 2:
            _ = a @ a  # a GEMM between launches
        o, l = zy.zyfa_fwd(tq, tk, tv, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, first) and torch.equal(l, flse), f"run {i} differs"
