"""GPU parity of partial-range attention (zyfa_fwd_range) and of the LSE
merge (zyfa_lse_merge) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from parity import (BF16_OUT_ABS, BF16_OUT_REL_ROUND, FP8_LSE_MAX, FP8_OUT_MAX, FP8_OUT_MEAN,
                    FP8_PRECISE_LSE_MAX, bf16_pair, check_bf16, check_partial, out_to_f64, tile_height)
from workloads import WORKLOADS, Workload, generate

pytestmark = pytest.mark.gpu

zy = pytest.importorskip("causal_flashattention_prefill_amd")


def _draw(B, Sq, Sk, H, Hk, dqk, layout, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = lambda s, h, d: (B, s, h, d) if layout == "bshd" else (B, h, s, d)
    q = rng.standard_normal(shp(Sq, H, dqk), dtype=np.float32)
    k = rng.standard_normal(shp(Sk, Hk, dqk), dtype=np.float32)
    v = rng.standard_normal(shp(Sk, Hk, 128), dtype=np.float32)
    return q, k, v


def _lse_rows(lse, layout):
    """LSE (B, H, S) rearranged to out's leading axes."""
    return np.swapaxes(lse, 1, 2) if layout == "bshd" else lse


CASES = [
    # B, Sq, Sk, q_pos0, k_pos0, H, Hk, dqk, layout
    (1, 300, 1000, 700, 0, 4, 2, 128, "bshd"),     # chunked prefill: last 300 rows over the prefix
    (2, 257, 520, 2000, 0, 2, 1, 128, "bshd"),     # keys wholly before the queries: no mask
    (1, 600, 300, 0, 200, 4, 4, 128, "bhsd"),      # keys start later: rows 0..199 see nothing
    (1, 100, 64, 0, 500, 2, 2, 128, "bshd"),       # no row sees a key
    (1, 520, 777, 300, 0, 2, 2, 192, "bhsd"),      # d_qk = 192
    (1, 700, 700, 37, 0, 3, 1, 128, "bshd"),       # offset not a tile multiple
    (1, 129, 1, 5, 5, 2, 1, 128, "bshd"),          # one key
    (1, 1000, 4097, 3097, 0, 2, 1, 192, "bshd"),   # several tiles each way, ragged
    (1, 300, 200, 2000, 0, 2, 1, 128, "bshd"),     # fewer than 256 keys, all before the queries
    (1, 520, 230, 5000, 0, 2, 2, 192, "bhsd"),     # the same at d_qk 192
]


@pytest.mark.parametrize("with_lse", [True, False])
@pytest.mark.parametrize("B,Sq,Sk,qp,kp,H,Hk,dqk,layout", CASES)
@pytest.mark.parametrize("tile_q", [256, 128])
def test_range_bf16(B, Sq, Sk, qp, kp, H, Hk, dqk, layout, with_lse, tile_q):
    print(f"case range bf16 B{B} Sq{Sq} Sk{Sk} q_pos0={qp} k_pos0={kp} H{H}/{Hk} d{dqk} {layout} lse={with_lse} "
          f"tile_q {tile_q}", flush=True)
    q, k, v = _draw(B, Sq, Sk, H, Hk, dqk, layout, 3000 + Sq + Sk)
    (tq, rq), (tk, rk), (tv, rv) = bf16_pair(q), bf16_pair(k), bf16_pair(v)
    with tile_height(zy, B, Sq, H, Hk, dqk, zy.DTYPE_BF16, tile_q):
        res = zy.zyfa_fwd_range(tq, tk, tv, qp, kp, layout=layout, return_lse=with_lse)
    torch.cuda.synchronize()
    out, lse = res if with_lse else (res, None)
    ro, rl = oracle.range_attention_ref(rq, rk, rv, qp, kp, layout=layout)
    l = None if lse is None else _lse_rows(lse.cpu().numpy().astype(np.float64), layout)
    check_partial(out_to_f64(out), ro, l, _lse_rows(rl, layout), f"range bf16 Sq{Sq} Sk{Sk} {qp}/{kp}")


def _fp8_inputs(q, k, v):
    """GPU quantize of each tensor, checked bit for bit against the oracle's;
    returns ([(codes, descale)] on the GPU, [oracle dequantized values])."""
    deq, dev = [], []
    for x in (q, k, v):
        t, r = bf16_pair(x)
        x8, ds = zy.zyfa_fp8_quantize(t)
        codes, d = oracle.fp8_quantize_ref(r)
        assert np.array_equal(x8.view(torch.uint8).cpu().numpy(), codes) and float(ds.item()) == float(d)
        deq.append(oracle.e4m3fn_decode(codes) * float(d))
        dev.append((x8, ds))
    return dev, deq


@pytest.mark.parametrize("B,Sq,Sk,qp,kp,H,Hk,dqk,layout", [CASES[i] for i in (0, 1, 2, 3, 4, 7, 8, 9)])
@pytest.mark.parametrize("tile_q,p_mode", [(256, "default"), (128, "default"), (128, "precise")])
def test_range_fp8(B, Sq, Sk, qp, kp, H, Hk, dqk, layout, tile_q, p_mode):
    print(f"case range fp8 B{B} Sq{Sq} Sk{Sk} q_pos0={qp} k_pos0={kp} H{H}/{Hk} d{dqk} {layout} tile_q {tile_q} "
          f"{p_mode}", flush=True)
    q, k, v = _draw(B, Sq, Sk, H, Hk, dqk, layout, 4000 + Sq + Sk)
    ((q8, qs), (k8, ks), (v8, vs)), deq = _fp8_inputs(q, k, v)
    with tile_height(zy, B, Sq, H, Hk, dqk, zy.DTYPE_FP8, tile_q):
        out, lse = zy.zyfa_fwd_range(q8, k8, v8, qp, kp, layout=layout, q_descale=qs, k_descale=ks, v_descale=vs,
                                     p_mode=p_mode)
    torch.cuda.synchronize()
    ro, rl = oracle.range_attention_ref(*deq, qp, kp, layout=layout)
    got_l = _lse_rows(lse.cpu().numpy().astype(np.float64), layout)
    # out and the LSE (from the rounded probabilities) at the FP8 bounds
    check_partial(out_to_f64(out), ro, got_l, _lse_rows(rl, layout), f"range fp8 Sq{Sq} Sk{Sk}", fp8=True)
    if p_mode == "precise":
        live = ~np.isneginf(_lse_rows(rl, layout))
        dl = np.abs(got_l - _lse_rows(rl, layout))[live]
        assert dl.size == 0 or dl.max() < FP8_PRECISE_LSE_MAX, f"max|dLSE|={dl.max():.3e}"


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("split", [100, 256, 611])
@pytest.mark.parametrize("p_mode", ["default", "precise"])
def test_fp8_split_and_merge_is_whole_attention(layout, split, p_mode):
    """FP8 keys [0, split) and [split, S) as two range calls (one descale per
    tensor, the codes split), merged on the GPU, against fp64 attention on
    the dequantized inputs over all keys: the merge is consistent because
    each partial's LSE comes from the same rounded probabilities as its
    output. Allowance: the FP8 gate plus the bf16 rounding of the two
    partial outputs carried through their weights."""
    B, S, H, Hk, dqk = 1, 700, 4, 2, 128
    print(f"case fp8 split-merge {layout} split={split} {p_mode}", flush=True)
    q, k, v = _draw(B, S, S, H, Hk, dqk, layout, 5100 + split)
    ((q8, qs), (k8, ks), (v8, vs)), (rq, rk, rv) = _fp8_inputs(q, k, v)
    ksl = (lambda x, a, b: x[:, a:b]) if layout == "bshd" else (lambda x, a, b: x[:, :, a:b])
    parts, refs = [], []
    for a, b in ((0, split), (split, S)):
        kk, vv = ksl(k8, a, b).contiguous(), ksl(v8, a, b).contiguous()
        parts.append(zy.zyfa_fwd_range(q8, kk, vv, 0, a, layout=layout, q_descale=qs, k_descale=ks, v_descale=vs,
                                       p_mode=p_mode))
        refs.append(oracle.range_attention_ref(rq, ksl(rk, a, b), ksl(rv, a, b), 0, a, layout=layout))
    out, lse = zy.zyfa_lse_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1], layout=layout)
    torch.cuda.synchronize()
    fo, fl = oracle.causal_attention_ref(rq, rk, rv, layout=layout)
    got, gl = out_to_f64(out), lse.cpu().numpy().astype(np.float64)
    (oa, la), (ob, lb) = refs
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    wa, wb = _lse_rows(wa / (wa + wb), layout)[..., None], _lse_rows(wb / (wa + wb), layout)[..., None]
    carry = BF16_OUT_REL_ROUND * (wa * np.abs(oa) + wb * np.abs(ob))
    d = np.abs(got - fo)
    bound = FP8_OUT_MAX + BF16_OUT_REL_ROUND * np.abs(fo) + carry
    print(f"fp8 split-merge: max|dout|={d.max():.3e} mean={d.mean():.2e} max|dLSE|={np.abs(gl - fl).max():.3e}",
          flush=True)
    assert np.all(d <= bound), f"max|dout|={d.max():.3e}"
    assert d.mean() <= FP8_OUT_MEAN, f"mean|dout|={d.mean():.3e}"
    lim = FP8_PRECISE_LSE_MAX if p_mode == "precise" else FP8_LSE_MAX
    assert np.all(np.abs(gl - fl) < lim), f"max|dLSE|={np.abs(gl - fl).max():.3e}"


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_whole_range_is_bitwise_zyfa_fwd(layout):
    w = WORKLOADS[1].resized(seqlen=700, name="r700")
    w = Workload(w.name, 1, 700, 4, 2, 128, 128, layout, ("bf16",), True, False, 11)
    q, k, v = generate(w)
    tq, tk, tv = (bf16_pair(x)[0] for x in (q, k, v))
    o1, l1 = zy.zyfa_fwd(tq, tk, tv, layout=layout, return_lse=True)
    o2, l2 = zy.zyfa_fwd_range(tq, tk, tv, 123, 123, layout=layout)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _synthetic_partials(B, S, H, layout, seed, empty_frac=0.1):
    """Seeded bf16 outputs and fp32 LSEs of two partial results, with some
    rows empty (-inf) in one or both."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = (B, S, H, 128) if layout == "bshd" else (B, H, S, 128)
    oa, ob = (rng.standard_normal(shp, dtype=np.float32) for _ in range(2))
    la, lb = (rng.normal(0.0, 4.0, (B, H, S)).astype(np.float32) for _ in range(2))
    la[rng.random((B, H, S)) < empty_frac] = -np.inf
    lb[rng.random((B, H, S)) < empty_frac] = -np.inf
    lb[0, 0, :3] = -np.inf
    la[0, 0, :3] = -np.inf                  # rows empty on both sides
    return oa, la, ob, lb


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,S,H", [(2, 333, 3)] + [tuple(int(x) for x in np.random.default_rng(40 + i).integers(
    [1, 1, 1], [4, 2000, 40])) for i in range(6)])
def test_merge_kernel_matches_oracle(layout, inplace, B, S, H):
    print(f"case merge {layout} inplace={inplace} B{B} S{S} H{H}", flush=True)
    oa, la, ob, lb = _synthetic_partials(B, S, H, layout, 21)
    (toa, roa), (tob, rob) = bf16_pair(oa), bf16_pair(ob)
    tla, tlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    if inplace:
        out, lse = zy.zyfa_lse_merge(toa, tla, tob, tlb, out=toa, lse=tla, layout=layout)
    else:
        out, lse = zy.zyfa_lse_merge(toa, tla, tob, tlb, layout=layout)
    torch.cuda.synchronize()
    ro, rl = oracle.lse_merge_layout_ref(roa, la.astype(np.float64), rob, lb.astype(np.float64), layout)
    got, gl = out_to_f64(out), lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), empty)
    assert np.all(got[_lse_rows(empty, layout)] == 0.0)
    # fp32 weights and sums (relative 1e-6), then one RNE to bf16 (2^-9 relative)
    d = np.abs(got - ro)
    assert np.all(d <= BF16_OUT_REL_ROUND * np.abs(ro) + 1e-5 * (np.abs(roa) + np.abs(rob))), d.max()
    fin = ~empty
    assert np.all(np.abs(gl[fin] - rl[fin]) <= 1e-5 + 1e-6 * np.abs(rl[fin]))


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
@pytest.mark.parametrize("split", [0, 100, 256, 611])
def test_split_and_merge_is_whole_attention(layout, split):
    """Keys [0, split) and [split, S) as two range calls, merged on the GPU,
    against the whole-sequence oracle. Allowance: the gate, plus the bf16
    rounding of the two partial outputs carried through their weights."""
    B, S, H, Hk = 1, 700, 4, 2
    print(f"case split-merge {layout} split={split}", flush=True)
    q, k, v = _draw(B, S, S, H, Hk, 128, layout, 5000 + split)
    (tq, rq), (tk, rk), (tv, rv) = bf16_pair(q), bf16_pair(k), bf16_pair(v)
    ksl = (lambda x, a, b: x[:, a:b]) if layout == "bshd" else (lambda x, a, b: x[:, :, a:b])
    parts, refs = [], []
    for a, b in ((0, split), (split, S)):
        if b == a:
            continue
        kk, vv = ksl(tk, a, b).contiguous(), ksl(tv, a, b).contiguous()
        parts.append(zy.zyfa_fwd_range(tq, kk, vv, 0, a, layout=layout))
        refs.append(oracle.range_attention_ref(rq, ksl(rk, a, b), ksl(rv, a, b), 0, a, layout=layout))
    if len(parts) == 1:
        out, lse = parts[0]
    else:
        out, lse = zy.zyfa_lse_merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1], layout=layout)
    torch.cuda.synchronize()
    fo, fl = oracle.causal_attention_ref(rq, rk, rv, layout=layout)
    got, gl = out_to_f64(out), lse.cpu().numpy().astype(np.float64)
    carry = 0.0
    if len(refs) == 2:
        (oa, la), (ob, lb) = refs
        m = np.maximum(la, lb)
        wa, wb = np.exp(la - m), np.exp(lb - m)
        wa, wb = _lse_rows(wa / (wa + wb), layout)[..., None], _lse_rows(wb / (wa + wb), layout)[..., None]
        carry = BF16_OUT_REL_ROUND * (wa * np.abs(oa) + wb * np.abs(ob))
    d = np.abs(got - fo)
    bound = BF16_OUT_ABS + BF16_OUT_REL_ROUND * np.abs(fo) + carry
    assert np.all(d <= bound), f"max|dout|={d.max():.3e}"
    assert np.all(np.abs(gl - fl) <= 1e-3), f"max|dLSE|={np.abs(gl - fl).max():.3e}"


def test_chunked_prefill_full_size_sampled_rows():
    """The last half of workload 2 (8192 tokens, GQA 32/8) as one chunk over
    the whole prefix, sampled rows against the oracle."""
    w = WORKLOADS[2]
    q, k, v = generate(w)
    Sq = w.seqlen // 2
    qc = np.ascontiguousarray(q[:, w.seqlen - Sq:])
    (tq, rq), (tk, rk), (tv, rv) = bf16_pair(qc), bf16_pair(k), bf16_pair(v)
    print(f"case chunked prefill {w.name} Sq{Sq} Sk{w.seqlen}", flush=True)
    out, lse = zy.zyfa_fwd_range(tq, tk, tv, w.seqlen - Sq, 0)
    torch.cuda.synchronize()
    o, l = out_to_f64(out), lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(2)
    for h in (0, 13, w.nheads - 1):
        rows = sorted(set([0, 1, 255, 256, Sq // 2, Sq - 1] + rng.integers(0, Sq, 10).tolist()))
        ro, rl = oracle.range_attention_rows_ref(rq, rk, rv, 0, h, rows, w.seqlen - Sq, 0)
        check_bf16(o[0, rows, h], ro, l[0, h, rows], rl, f"chunk head {h}")
