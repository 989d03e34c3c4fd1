"""GPU results against closed forms, without the oracle: when every score of
a row is the same (all keys equal, or q = 0), causal softmax weights are
uniform, so output row i is the mean of v_0 .. v_i and the LSE is
s + ln(i + 1) ("ZYFA" README, Usage: causal attention with the natural-log
LSE). In FP8 every such probability is exactly 1 (exact P rounds 2^0 to the
code of 1; lean P writes the code RNE(8 * 0 + C) = 56, also 1), so the
weights stay exactly uniform and only the fp32 sums and the bf16 output
rounding remain.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import FP8_MFMA_REL, out_to_f64

pytestmark = pytest.mark.gpu

zy = pytest.importorskip("causal_flashattention_prefill_amd")


def _prefix_mean(v):
    """(S, d) -> (S, d): row i is the mean of rows 0..i, in float64."""
    return np.cumsum(v, axis=0) / np.arange(1, v.shape[0] + 1)[:, None]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("which", ["equal_keys", "zero_queries"])
@pytest.mark.parametrize("B,S,H,Hk,dqk,layout", [(1, 1000, 4, 2, 128, "bshd"), (2, 333, 2, 2, 192, "bhsd")])
def test_uniform_rows_give_the_prefix_mean(B, S, H, Hk, dqk, layout, which, dtype):
    rng = np.random.default_rng(5000 + S + dqk + 7 * (which == "zero_queries") + 13 * (dtype == "fp8"))
    shape = (lambda h, d: (B, S, h, d)) if layout == "bshd" else (lambda h, d: (B, h, S, d))
    q = rng.standard_normal(shape(H, dqk)).astype(np.float32)
    k = rng.standard_normal(shape(Hk, dqk)).astype(np.float32)
    v = rng.standard_normal(shape(Hk, 128)).astype(np.float32)
    if which == "equal_keys":
        sel = (slice(None), slice(0, 1)) if layout == "bshd" else (slice(None), slice(None), slice(0, 1))
        k[...] = k[sel]                        # every position carries the first key of its head
    else:
        q[...] = 0.0
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    print(f"case closed form {which} {dtype} B{B} S{S} H{H}/{Hk} d{dqk} {layout}", flush=True)
    kw = dict(layout=layout, return_lse=True)
    if dtype == "fp8":
        (tq, qs), (tk, ks), (tv, vs) = (zy.zyfa_fp8_quantize(x) for x in (tq, tk, tv))
        kw.update(q_descale=qs, k_descale=ks, v_descale=vs)
        torch.cuda.synchronize()
        vals = [oracle.e4m3fn_decode(t.view(torch.uint8).cpu().numpy()) * float(s.item())
                for t, s in ((tq, qs), (tk, ks), (tv, vs))]
    else:
        vals = [t.float().cpu().numpy().astype(np.float64) for t in (tq, tk, tv)]
    out, lse = zy.zyfa_fwd(tq, tk, tv, **kw)
    torch.cuda.synchronize()
    o = out_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    qv, kv, vv = vals
    g = H // Hk
    scale = 1.0 / np.sqrt(dqk)
    hv = (lambda x: np.swapaxes(x, 1, 2)) if layout == "bshd" else (lambda x: x)
    Q, K, V, O = hv(qv), hv(kv), hv(vv), hv(o)
    for b in range(B):
        for h in range(H):
            want = _prefix_mean(V[b, h // g])
            got = O[b, h]
            # bf16 output: half an ulp of each value, plus the fp32 sums (and,
            # in FP8, the matrix instruction's own summation error)
            ab = 1e-4 if dtype == "fp8" else 1e-5
            assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + ab), \
                f"b{b} h{h}: max {np.abs(got - want).max():.3e}"
            k0, qh = K[b, h // g][0], Q[b, h]
            s = (qh @ k0) * scale                              # the one score of each row
            want_lse = s + np.log(np.arange(1, S + 1))
            # fp32 sums; in FP8 the score also carries the FP8 instruction's
            # error, at most FP8_MFMA_REL of sum_c |q_c k_c| (times the scale)
            tol = 1e-5 + 1e-6 * np.abs(want_lse)
            if dtype == "fp8":
                tol = tol + FP8_MFMA_REL * scale * (np.abs(qh) @ np.abs(k0))
            assert np.all(np.abs(l[b, h] - want_lse) <= tol), \
                f"b{b} h{h}: lse max {np.abs(l[b, h] - want_lse).max():.3e}"
