"""Bitwise run-to-run determinism at full size, and the quantizer's
independence from other streams ("ZYFA" README, Accuracy: outputs are
identical in every launch, also with a GEMM running between them).

Every output tile is written by one workgroup that visits its keys in a
fixed order, with no atomics, so repeated launches must agree bit for bit:
each workload at its full size, in each dtype it names (and the precise FP8
mode where it exists), three launches with a GEMM between them, the last on
another stream; out and LSE compared with torch.equal.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import bf16_pair
from workloads import WORKLOADS, generate

pytestmark = pytest.mark.gpu

zy = pytest.importorskip("causal_flashattention_prefill_amd")

CASES = [(1, "bf16", "default"), (2, "bf16", "default"), (3, "fp8", "default"), (3, "fp8", "precise"),
         (4, "bf16", "default"), (4, "fp8", "default"), (5, "bf16", "default"), (5, "fp8", "default"),
         (5, "fp8", "precise")]


@pytest.mark.parametrize("wid,dtype,p_mode", CASES)
def test_full_size_repeats_are_bitwise_equal(wid, dtype, p_mode):
    w = WORKLOADS[wid]
    print(f"case determinism {w.name} {dtype} {p_mode} lse={w.with_lse}", flush=True)
    q, k, v = generate(w)
    tq, tk, tv = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in (q, k, v))
    del q, k, v
    kw = dict(layout=w.layout, return_lse=w.with_lse)
    if dtype == "fp8":
        (tq, qs), (tk, ks), (tv, vs) = (zy.zyfa_fp8_quantize(x) for x in (tq, tk, tv))
        kw.update(q_descale=qs, k_descale=ks, v_descale=vs, p_mode=p_mode)
    a = torch.randn(4096, 4096, device="cuda")
    runs = []
    side = torch.cuda.Stream()
    for i in range(3):
        _ = a @ a
        if i < 2:
            r = zy.zyfa_fwd(tq, tk, tv, **kw)
        else:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                r = zy.zyfa_fwd(tq, tk, tv, **kw)
            torch.cuda.current_stream().wait_stream(side)
        runs.append(r if isinstance(r, tuple) else (r, None))
    torch.cuda.synchronize()
    o0, l0 = runs[0]
    assert torch.isfinite(o0.float()).all()
    for i, (o, l) in enumerate(runs[1:], 1):
        assert torch.equal(o, o0), f"run {i}: out differs"
        if l0 is not None:
            assert torch.equal(l, l0), f"run {i}: lse differs"


def test_quantize_on_two_streams_concurrently():
    """Two streams quantize different tensors at the same time, many times;
    every result must equal the oracle's codes and descale bit for bit (the
    quantizer keeps its partial maxima in the call's own output, so
    concurrent calls cannot mix them)."""
    rng = np.random.default_rng(44)
    xs = [(rng.standard_normal(3_000_000) * s).astype(np.float32) for s in (1.0, 300.0)]
    pairs = [bf16_pair(x) for x in xs]
    refs = [oracle.fp8_quantize_ref(r) for _, r in pairs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    n = 20
    outs = [[(torch.empty(t.shape, dtype=torch.float8_e4m3fn, device="cuda"),
              torch.empty(1, dtype=torch.float32, device="cuda")) for _ in range(n)] for t, _ in pairs]
    print("case quantize on two streams", flush=True)
    torch.cuda.synchronize()
    for i in range(n):
        for j, s in enumerate(streams):
            with torch.cuda.stream(s):
                zy.zyfa_fp8_quantize(pairs[j][0], outs[j][i][0], outs[j][i][1], stream=s)
    torch.cuda.synchronize()
    for j in range(2):
        codes, d = refs[j]
        for i in range(n):
            x8, ds = outs[j][i]
            assert float(ds.item()) == float(d), f"stream {j} call {i}: descale {ds.item()} vs {d}"
            assert np.array_equal(x8.view(torch.uint8).cpu().numpy(), codes), f"stream {j} call {i}: codes differ"
