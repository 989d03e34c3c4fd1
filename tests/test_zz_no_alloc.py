"""zyfa_fwd_noalloc through the C ABI: the variant of zyfa_fwd_ex that
allocates nothing (its job table goes into the library's static device
buffer). Its output must equal zyfa_fwd_ex's bit for bit: each output tile
is computed the same way whichever workgroup takes it, and the table is the
same. Two calls in a row, the second with a smaller input (the buffer keeps
the first call's table, which the second overwrites in part), per dtype and
mode; a shape whose table exceeds the buffer is refused; and the call
captured in a graph on a shape that was never prepared replays equal to the
eager result."""
import numpy as np
import pytest
import torch

from parity import bf16_pair
from workloads import Workload, generate

pytestmark = pytest.mark.gpu

zy = pytest.importorskip("causal_flashattention_prefill_amd")


def _inputs(w, dtype):
    q, k, v = generate(w)
    t = [bf16_pair(x)[0] for x in (q, k, v)]
    if dtype == "bf16":
        return t, {}
    (q8, qs), (k8, ks), (v8, vs) = (zy.zyfa_fp8_quantize(x) for x in t)
    return [q8, k8, v8], dict(q_descale=qs, k_descale=ks, v_descale=vs)


def _out_like(w):
    shape = (w.batch, w.seqlen, w.nheads, w.d_v) if w.layout == "bshd" else (w.batch, w.nheads, w.seqlen, w.d_v)
    return (torch.empty(shape, dtype=torch.bfloat16, device="cuda"),
            torch.empty((w.batch, w.nheads, w.seqlen), dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("dtype,p_mode", [("bf16", "default"), ("fp8", "default"), ("fp8", "exact"),
                                          ("fp8", "precise")])
def test_noalloc_equals_fwd_ex_on_two_calls(dtype, p_mode):
    shapes = [Workload("na_big", 2, 3000, 16, 4, 128, 128, "bshd", (dtype,), True, False, 301),
              Workload("na_small", 1, 333, 4, 1, 192, 128, "bhsd", (dtype,), True, False, 302)]
    for w in shapes:
        print(f"case noalloc {dtype} {p_mode} B{w.batch} S{w.seqlen} H{w.nheads}/{w.nheads_k} d{w.d_qk}", flush=True)
        (q, k, v), kw = _inputs(w, dtype)
        out, lse = _out_like(w)
        zy.zyfa_fwd_noalloc(q, k, v, out, lse, layout=w.layout, p_mode=p_mode, **kw)
        ref, ref_lse = zy.zyfa_fwd(q, k, v, layout=w.layout, return_lse=True, p_mode=p_mode, **kw)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out, ref), f"{w.name}: out differs from zyfa_fwd_ex"
        assert torch.equal(lse, ref_lse), f"{w.name}: lse differs from zyfa_fwd_ex"


def test_noalloc_refuses_a_table_beyond_the_buffer():
    L = zy.lib()
    # 64 x 64 heads x 64 pairs = 262144 jobs > 65536 entries; pointers are
    # never dereferenced (the check comes before any launch)
    rc = L.zyfa_fwd_noalloc(256, 256, 256, 256, None, 64, 32768, 64, 8, 128, 128, 0, 0, None, None, None, 0.0, 0,
                            None)
    assert rc == zy.STATUS["ZYFA_ERR_SCRATCH"]


def test_noalloc_captured_without_prepare():
    w = Workload("na_graph", 1, 777, 4, 2, 128, 128, "bshd", ("bf16",), True, False, 303)
    (q, k, v), _ = _inputs(w, "bf16")
    out, lse = _out_like(w)
    ref, ref_lse = _out_like(w)
    zy.zyfa_release()     # no plan for any shape
    zy.zyfa_fwd_noalloc(q, k, v, ref, ref_lse)
    torch.cuda.synchronize()
    zy.zyfa_release()
    print("case noalloc under capture B1 S777 H4/2 d128", flush=True)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        zy.zyfa_fwd_noalloc(q, k, v, out, lse, stream=s)
    for i in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), f"replay {i} differs"
