"""Tensors past 4 GiB, and (batch, head) slices past 4 GiB, through the C ABI.

With 65536 heads of d = 128 in bshd, one position of q spans 16 MiB, so the
300 rows of a head reach 4.7 GiB past the tensor's base: every 32-bit byte
offset from a slice base would wrap. In bhsd the same tensor is 4.7 GiB with
small slices, which exercises the 64-bit head and batch bases. Only a few
heads carry random values (the rest are zero); their outputs are compared
with the oracle, including the last head, whose rows lie furthest out.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import bf16_pair, check_bf16, check_fp8, out_to_f64
from workloads import sampled_heads

pytestmark = pytest.mark.gpu

zy = pytest.importorskip("causal_flashattention_prefill_amd")

S, H, D = 300, 65536, 128
HEADS = [0, 1, 40961, H - 2, H - 1]


def _big_inputs(layout: str, seed: int):
    q, k, v = sampled_heads(seed, S, HEADS, D, D)
    shape = (1, S, H, D) if layout == "bshd" else (1, H, S, D)
    tens, refs = [], []
    for x in (q, k, v):
        t = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        ref = []
        for i, h in enumerate(HEADS):
            src, r = bf16_pair(x[i])   # torch's cast and the oracle's agree bit for bit
            if layout == "bshd":
                t[0, :, h] = src
            else:
                t[0, h] = src
            ref.append(r)
        tens.append(t)
        refs.append(np.stack(ref))
    return tens, refs


def _head_out(t: torch.Tensor, layout: str, h: int) -> np.ndarray:
    return out_to_f64(t[0, :, h] if layout == "bshd" else t[0, h])


@pytest.mark.parametrize("layout", ["bshd", "bhsd"])
def test_bf16_past_4gib(layout):
    print(f"case large bf16 {layout} S{S} H{H} d{D}", flush=True)
    (tq, tk, tv), (rq, rk, rv) = _big_inputs(layout, 77)
    assert tq.numel() * tq.element_size() > 4 * 2**30
    out, lse = zy.zyfa_fwd(tq, tk, tv, layout=layout, return_lse=True)
    torch.cuda.synchronize()
    l = lse.cpu().numpy().astype(np.float64)
    for i, h in enumerate(HEADS):
        ro, rl = oracle.causal_attention_ref(rq[i][None, :, None], rk[i][None, :, None], rv[i][None, :, None])
        check_bf16(_head_out(out, layout, h), ro[0, :, 0], l[0, h], rl[0, 0], f"large {layout} head {h}")
    del tq, tk, tv, out, lse
    torch.cuda.empty_cache()


def test_fp8_past_4gib():
    layout = "bshd"
    print(f"case large fp8 {layout} S{S} H{H} d{D}", flush=True)
    (tq, tk, tv), (rq, rk, rv) = _big_inputs(layout, 78)
    deq = []
    pairs = []
    for t, r in ((tq, rq), (tk, rk), (tv, rv)):
        x8, ds = zy.zyfa_fp8_quantize(t)
        # the other heads are zero, so the whole tensor's amax is that of the
        # sampled heads, and the oracle quantizes those on its own
        codes, descale = oracle.fp8_quantize_ref(r)
        assert float(ds.item()) == descale
        for i, h in enumerate(HEADS):
            got = (x8[0, :, h] if layout == "bshd" else x8[0, h]).view(torch.uint8).cpu().numpy()
            assert np.array_equal(got, codes[i]), f"codes of head {h} differ"
        deq.append(oracle.e4m3fn_decode(codes) * descale)
        pairs.append((x8, ds))
        del t
    (q8, qs), (k8, ks), (v8, vs) = pairs
    del tq, tk, tv
    out = zy.zyfa_fwd(q8, k8, v8, layout=layout, q_descale=qs, k_descale=ks, v_descale=vs)
    torch.cuda.synchronize()
    got = np.concatenate([_head_out(out, layout, h) for h in HEADS])
    ref = np.concatenate([oracle.causal_attention_ref(deq[0][i][None, :, None], deq[1][i][None, :, None],
                                                      deq[2][i][None, :, None])[0][0, :, 0]
                          for i in range(len(HEADS))])
    check_fp8(got, ref, "large fp8")
    del q8, k8, v8, out
    torch.cuda.empty_cache()
