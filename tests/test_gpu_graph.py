"""The C ABI under HIP graph capture: once the plan of a shape exists,
zyfa_fwd, zyfa_fwd_range, zyfa_lse_merge (and zyfa_fp8_quantize always)
allocate nothing and copy nothing from the host, so they can be captured;
every replay must reproduce the eager results bit for bit, with eager work
and synchronizations between replays. A call that would have to build a
plan under capture returns ZYFA_ERR_CAPTURE without enqueueing anything
("ZYFA" README, Usage: run each new shape once before capturing), and the
stream stays usable."""
import numpy as np
import pytest
import torch

from parity import bf16_pair
from workloads import Workload, generate

pytestmark = pytest.mark.gpu

zy = pytest.importorskip("causal_flashattention_prefill_amd")


def test_graph_replays_match_eager():
    w = Workload("graph", 1, 700, 4, 2, 128, 128, "bshd", ("bf16", "fp8"), True, False, 91)
    q, k, v = generate(w)
    tq, tk, tv = (bf16_pair(x)[0] for x in (q, k, v))
    print("case graph capture B1 S700 H4/2 d128", flush=True)
    # eager results (also builds the plans)
    out_e, lse_e = zy.zyfa_fwd(tq, tk, tv, return_lse=True)
    (q8e, qse), (k8e, kse), (v8e, vse) = (zy.zyfa_fp8_quantize(x) for x in (tq, tk, tv))
    out8_e = zy.zyfa_fwd(q8e, k8e, v8e, q_descale=qse, k_descale=kse, v_descale=vse)
    h = w.seqlen // 2
    ka, va = tk[:, :h].contiguous(), tv[:, :h].contiguous()
    kb, vb = tk[:, h:].contiguous(), tv[:, h:].contiguous()
    pa = zy.zyfa_fwd_range(tq, ka, va, 0, 0)
    pb = zy.zyfa_fwd_range(tq, kb, vb, 0, h)
    om_e, lm_e = zy.zyfa_lse_merge(pa[0], pa[1], pb[0], pb[1])
    torch.cuda.synchronize()

    # static buffers written by the graph
    out_g, lse_g = torch.empty_like(out_e), torch.empty_like(lse_e)
    q8, k8, v8 = torch.empty_like(q8e), torch.empty_like(k8e), torch.empty_like(v8e)
    qs, ks, vs = (torch.empty_like(qse) for _ in range(3))
    out8_g = torch.empty_like(out8_e)
    oa, la = torch.empty_like(pa[0]), torch.empty_like(pa[1])
    ob, lb = torch.empty_like(pb[0]), torch.empty_like(pb[1])
    om_g, lm_g = torch.empty_like(om_e), torch.empty_like(lm_e)

    def work():
        zy.zyfa_fwd(tq, tk, tv, out_g, lse_g)
        for x, x8, xs in ((tq, q8, qs), (tk, k8, ks), (tv, v8, vs)):
            zy.zyfa_fp8_quantize(x, x8, xs)
        zy.zyfa_fwd(q8, k8, v8, out8_g, q_descale=qs, k_descale=ks, v_descale=vs)
        zy.zyfa_fwd_range(tq, ka, va, 0, 0, oa, la)
        zy.zyfa_fwd_range(tq, kb, vb, 0, h, ob, lb)
        zy.zyfa_lse_merge(oa, la, ob, lb, om_g, lm_g)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    a = torch.randn(1024, 1024, device="cuda")
    for i in range(4):
        for t in (out_g, lse_g, q8.view(torch.uint8), out8_g, om_g, lm_g):
            t.zero_()                         # eager work between replays
        _ = a @ a
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(lse_g, lse_e), f"replay {i}: bf16 differs"
        assert torch.equal(q8.view(torch.uint8), q8e.view(torch.uint8)) and torch.equal(qs, qse), f"replay {i}: quantize"
        assert torch.equal(out8_g, out8_e), f"replay {i}: fp8 differs"
        assert torch.equal(om_g, om_e) and torch.equal(lm_g, lm_e), f"replay {i}: range/merge differs"


def test_unprepared_shape_under_capture_returns_capture_error():
    w = Workload("capture", 1, 333, 4, 2, 128, 128, "bshd", ("bf16", "fp8"), True, False, 92)
    q, k, v = generate(w)
    tq, tk, tv = (bf16_pair(x)[0] for x in (q, k, v))
    (q8, qs), (k8, ks), (v8, vs) = (zy.zyfa_fp8_quantize(x) for x in (tq, tk, tv))
    out = torch.empty((1, 333, 4, 128), dtype=torch.bfloat16, device="cuda")
    zy.zyfa_release()      # no plan exists for any shape now
    torch.cuda.synchronize()
    print("case capture error path B1 S333 H4/2 d128", flush=True)
    errors = []
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for call in (lambda: zy.zyfa_prepare(1, 333, 4, 2, 128, 128, stream=s),
                     lambda: zy.zyfa_fwd(tq, tk, tv, out, stream=s),
                     lambda: zy.zyfa_fwd(q8, k8, v8, out, q_descale=qs, k_descale=ks, v_descale=vs,
                                         p_mode="precise", stream=s),
                     lambda: zy.zyfa_fwd_range(tq, tk, tv, 0, 0, out, stream=s)):
            try:
                call()
            except zy.ZyfaError as e:
                errors.append(e.status)
        zy.zyfa_fp8_quantize(tq, q8, qs, stream=s)   # needs no plan: captured
    assert errors == [zy.STATUS["ZYFA_ERR_CAPTURE"]] * 4, errors
    # the stream (and the library) stay usable: prepare, then the same calls
    zy.zyfa_prepare(1, 333, 4, 2, 128, 128, dtype=zy.DTYPE_FP8, stream=s)
    zy.zyfa_prepare(1, 333, 4, 2, 128, 128, stream=s)
    with torch.cuda.stream(s):
        o1 = zy.zyfa_fwd(tq, tk, tv, stream=s)
        o2 = zy.zyfa_fwd(q8, k8, v8, q_descale=qs, k_descale=ks, v_descale=vs, p_mode="precise", stream=s)
    s.synchronize()
    ref = zy.zyfa_fwd(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(o1, ref) and torch.isfinite(o2.float()).all()
    g.replay()       # the captured quantize alone
    torch.cuda.synchronize()
