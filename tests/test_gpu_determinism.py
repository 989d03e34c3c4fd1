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


def test_attention_on_two_streams_concurrently():
    """Two host threads, each on its own stream, run attention on different
    shapes (BF16 d 128 GQA with the LSE on the automatic 128-row tiles; FP8
    d_qk 192 set to 256-row tiles) at the same time, right after
    zyfa_release, so both build their plans concurrently under the library's
    lock and their persistent grids share the GPU. Every result must equal
    the same call run alone, bit for bit."""
    import threading
    rng = np.random.default_rng(45)
    zy.zyfa_set_tile_q(1, 2500, 16, 16, d_qk=192, dtype=zy.DTYPE_FP8, tile_q=256)

    def bf16(shape, s=1.0):
        return torch.from_numpy((rng.standard_normal(shape) * s).astype(np.float32)).to(torch.bfloat16).cuda()

    qa, ka, va = bf16((1, 3000, 8, 128)), bf16((1, 3000, 2, 128)), bf16((1, 3000, 2, 128))
    qb, kb, vb = bf16((1, 16, 2500, 192)), bf16((1, 16, 2500, 192)), bf16((1, 16, 2500, 128))
    (qb8, dq), (kb8, dk), (vb8, dv) = (zy.zyfa_fp8_quantize(x) for x in (qb, kb, vb))
    calls = [lambda out, lse, s: zy.zyfa_fwd(qa, ka, va, out, lse, stream=s),
             lambda out, lse, s: zy.zyfa_fwd(qb8, kb8, vb8, out, None, layout="bhsd", q_descale=dq, k_descale=dk,
                                             v_descale=dv, stream=s)]
    shapes = [((1, 3000, 8, 128), (1, 8, 3000)), ((1, 16, 2500, 128), None)]
    print("case attention on two streams", flush=True)
    refs = []
    for f, (os_, ls) in zip(calls, shapes):
        o = torch.empty(os_, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(ls, dtype=torch.float32, device="cuda") if ls else None
        f(o, lse, torch.cuda.current_stream())
        refs.append((o, lse))
    torch.cuda.synchronize()
    n = 6
    outs = [[(torch.empty(os_, dtype=torch.bfloat16, device="cuda"),
              torch.empty(ls, dtype=torch.float32, device="cuda") if ls else None) for _ in range(n)]
            for os_, ls in shapes]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    errors = []

    def worker(j):
        try:
            with torch.cuda.stream(streams[j]):
                for i in range(n):
                    calls[j](outs[j][i][0], outs[j][i][1], streams[j])
        except Exception as e:   # reported by the main thread
            errors.append(e)

    zy.zyfa_release()
    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    zy.zyfa_set_tile_q(1, 2500, 16, 16, d_qk=192, dtype=zy.DTYPE_FP8, tile_q=0)
    for j in range(2):
        ro, rl = refs[j]
        for i in range(n):
            o, lse = outs[j][i]
            assert torch.equal(o, ro), f"shape {j} call {i}: out differs"
            if rl is not None:
                assert torch.equal(lse, rl), f"shape {j} call {i}: lse differs"
