"""Throughput of causal prefill attention on one MI355X, one JSON line.

The headline (`value`, `ms_per_step`, `roofline`) is one step of the hot
path on the MLA-prefill workload: one BF16 attention launch on batch 1,
seqlen 16384, 16 heads, d_qk 192 / d_v 128, bhsd, timed as the average of
`--steps` back-to-back launches. Every other case (BF16 and FP8 GQA at 16K
tokens with the FP8 quantizer timed separately, FP8 at d_qk 192, the
precise FP8 mode, workload 5, one GPU's share, partial-range calls, the LSE
merge, the README's own configuration) is timed the same way and reported
under `config.cases`; none of them is part of `ms_per_step`. Inputs are
resident in HBM before timing starts. Each launch is bracketed by HIP
events on the stream it runs on. Before its W warm-up and K timed steps,
every case first runs back to back for --settle-seconds (1 s by default,
the warm-up of the README's sustained protocol): right after the GPU has
been idle, the first tens of launches of the 16K cases run up to 20 %
slower than the steady state while the board leaves its idle power state,
and 5 warm-up launches (5 ms) do not cover that.

Throughput is causal TFLOP/s = B * H * S^2 * (d_qk + d_v) / time, the
count of the "ZYFA" README's kernel-benchmark protocol.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X published dense MFMA peaks

# name -> (workload number, dtype); workloads are defined in workloads/.
CASES = {
    "bf16_d192_s16384": (4, "bf16"),
    "bf16_d128_gqa_s16384": (3, "bf16"),
    "fp8_d128_gqa_s16384": (3, "fp8"),
    "fp8_d192_s16384": (4, "fp8"),
    "fp8_d128_share8_s16384": (3, "fp8"),
    "fp8_d192_lean_s16384": (4, "fp8"),
    "fp8_d128_gqa_precise_s16384": (3, "fp8"),
    "bf16_act_s32000_b2": (5, "bf16"),
    "fp8_act_s32000_b2": (5, "fp8"),
    "fp8_act_precise_s32000_b2": (5, "fp8"),
}
# Cases run with a non-default FP8 probability mode: workload 4 with lean P
# (the README keeps exact P at d_qk = 192; lean P is the library's option),
# and the precise mode (bf16-MFMA scores, P split into two e4m3 parts; the
# mode that meets the FP8 gate on workload 5's activation-like inputs).
PMODE = {"fp8_d192_lean_s16384": "lean", "fp8_d128_gqa_precise_s16384": "precise",
         "fp8_act_precise_s32000_b2": "precise"}
# Cases reported without the quantizer timing and the sustained-clock runs.
EXTRA = {"bf16_act_s32000_b2", "fp8_act_s32000_b2"}
# Cases run on a resized workload: one GPU's share of workload 3 when its
# heads are split over 8 GPUs in whole GQA groups (4 query heads over 1 KV
# head, 16384 tokens): the kernel at the shape each GPU would run.
RESIZED = {"fp8_d128_share8_s16384": {"nheads": 4, "nheads_k": 1, "name": "gqa_fp8_s16384_share8"}}
# Partial-range calls and the LSE merge, on the workload-3 shape (batch 1,
# 16384 keys, 32 / 8 heads, d 128, bshd): the last 4096 queries as one chunk
# over the whole prefix (chunked prefill, LSE returned), and the merge of two
# partial results of all 16384 rows (HBM-bound).
RANGE_CASES = {
    "bf16_chunk4096_s16384": "bf16",
    "fp8_chunk4096_s16384": "fp8",
}
CHUNK_Q = 4096
# The README's own benchmark configuration (Performance, kernel-benchmark
# protocol): causal MHA, batch 1, max(32, 262144 / S) heads (128 at 2K, 32 at
# 16K and 32K), q, k, v Gaussian with standard deviation 0.1, bshd. Reported
# beside the README's MI355X figure for the same configuration (another
# software stack and board: context, not the target). (dtype, d_qk, S, TF/s)
CONTEXT_CASES = {
    "ctx_bf16_d128_std01_s16384": ("bf16", 128, 16384, 1237.0),
    "ctx_bf16_d192_std01_s16384": ("bf16", 192, 16384, 1296.0),
    "ctx_fp8_d128_std01_s16384": ("fp8", 128, 16384, 2597.0),
    "ctx_fp8_d192_std01_s16384": ("fp8", 192, 16384, 2391.0),
    "ctx_bf16_d128_std01_s2048": ("bf16", 128, 2048, 1000.0),
    "ctx_bf16_d192_std01_s2048": ("bf16", 192, 2048, 1008.0),
    "ctx_fp8_d128_std01_s2048": ("fp8", 128, 2048, 1942.0),
    "ctx_fp8_d192_std01_s2048": ("fp8", 192, 2048, 1929.0),
    "ctx_bf16_d128_std01_s32768": ("bf16", 128, 32768, 1265.0),
    "ctx_bf16_d192_std01_s32768": ("bf16", 192, 32768, 1330.0),
    "ctx_fp8_d128_std01_s32768": ("fp8", 128, 32768, 2672.0),
    "ctx_fp8_d192_std01_s32768": ("fp8", 192, 32768, 2464.0),
}
MERGE_CASE = "merge_bf16_s16384"
HBM_PEAK_GBS = 8000.0
HEADLINE = "bf16_d192_s16384"
DESCRIPTIONS = {
    "bf16_d192_s16384": "causal MLA-prefill form, bf16: batch 1, seqlen 16384, nheads 16 = nheads_k, d_qk 192, "
                        "d_v 128, bhsd, q/k/v N(0,1)",
    "bf16_d128_gqa_s16384": "causal GQA, bf16: batch 1, seqlen 16384, nheads 32, nheads_k 8, d 128, bshd, N(0,1)",
    "fp8_d128_gqa_s16384": "causal GQA, fp8 e4m3 per-tensor pow2 descales: batch 1, seqlen 16384, nheads 32, "
                           "nheads_k 8, d 128, bshd, N(0,1)",
    "fp8_d192_s16384": "causal MLA-prefill form, fp8 e4m3: batch 1, seqlen 16384, nheads 16, d_qk 192, d_v 128, "
                       "bhsd, N(0,1)",
    "fp8_d128_share8_s16384": "one GPU's share of the fp8 GQA case over 8 GPUs: batch 1, seqlen 16384, nheads 4, "
                              "nheads_k 1, d 128, bshd, N(0,1)",
    "fp8_d192_lean_s16384": "causal MLA-prefill form, fp8 e4m3 with lean P: batch 1, seqlen 16384, nheads 16, "
                            "d_qk 192, d_v 128, bhsd, N(0,1)",
    "fp8_d128_gqa_precise_s16384": "causal GQA, fp8 e4m3, precise mode (bf16-MFMA scores, hi + lo P): batch 1, "
                                   "seqlen 16384, nheads 32, nheads_k 8, d 128, bshd, N(0,1)",
    "bf16_act_s32000_b2": "causal GQA, bf16, activation-like q/k: batch 2, seqlen 32000, nheads 32, nheads_k 8, "
                          "d 128, bshd",
    "fp8_act_s32000_b2": "causal GQA, fp8 e4m3 (default mode, known accuracy limit on these inputs), "
                         "activation-like q/k: batch 2, seqlen 32000, nheads 32, nheads_k 8, d 128, bshd",
    "fp8_act_precise_s32000_b2": "causal GQA, fp8 e4m3 precise mode, activation-like q/k: batch 2, seqlen 32000, "
                                 "nheads 32, nheads_k 8, d 128, bshd",
}
ALL_CASES = list(CASES) + list(RANGE_CASES) + [MERGE_CASE] + list(CONTEXT_CASES)


def range_flops(B, H, Sq, Sk, delta, dqk, dv):
    """2 (d_qk + d_v) FLOPs per visible (query, key) pair; key c visible to
    row r when c <= r + delta. For whole-sequence causal attention this is
    S (S + 1) (d_qk + d_v) per head, the README's count up to the diagonal."""
    import numpy as np
    r = np.arange(Sq, dtype=np.float64)
    pairs = np.clip(r + delta + 1, 0, Sk).sum()
    return 2.0 * (dqk + dv) * B * H * pairs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", default="", help="comma-separated subset of: " + ",".join(ALL_CASES))
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a reference for HBM byte counters)")
    ap.add_argument("--protocol-a", action="store_true",
                    help="only the README configuration cases, timed with the README's kernel-benchmark protocol")
    ap.add_argument("--sustain-seconds", type=float, default=3.0,
                    help="seconds per timed run of the sustained-clock protocol on each 16K gate case (0: skip)")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="seconds of back-to-back launches before each case's warm-up and timed steps")
    return ap.parse_args()


# Sources that decide the code and launch shape of each attention kernel; a
# stored counter reading is used only while their hash is unchanged.
PKG = os.path.join(ROOT, "causal_flashattention_prefill_amd", "csrc")
COMMON_SOURCES = ["device_common.h", "zyfa_internal.h", "api.cpp", "plan.cpp", "plan.h"]
KERNEL_SOURCES = {"bf16": ["attn_bf16.hip"] + COMMON_SOURCES, "fp8": ["attn_fp8.hip"] + COMMON_SOURCES}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash(dtype: str) -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    that a comment edit keeps a stored reading valid and a code edit does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[dtype]:
        with open(os.path.join(PKG, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(f.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def stored_traffic(name: str, dtype: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE
    reading of this case, each divided by the factor the same counter showed
    for a plain copy of known size; None when there is no reading or the
    kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)[name]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash(dtype):
        return None
    return rec["fetch_kib"] * 1024 / rec["copy_fetch_factor"] + rec["write_kib"] * 1024 / rec["copy_write_factor"]


class PowerClockSampler:
    """Samples the GFX clock and socket power of the GPU behind cuda:0 with
    amdsmi from a host thread; empty readings if amdsmi is unavailable."""

    def __init__(self, period_s: float = 0.05):
        import threading
        self.period, self.clk, self.pw, self.err = period_s, [], [], None
        self._stop = threading.Event()
        self._thr = threading.Thread(target=self._run, daemon=True)
        self._handle = None
        try:
            import amdsmi
            import torch
            amdsmi.amdsmi_init()
            props = torch.cuda.get_device_properties(0)
            want = (getattr(props, "pci_domain_id", 0), props.pci_bus_id, props.pci_device_id)
            for hnd in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(hnd)  # "dddd:bb:dd.f"
                dom, bus, devfn = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(devfn.split(".")[0], 16)) == want:
                    self._handle = hnd
            if self._handle is None:
                self.err = "no amdsmi device matches cuda:0"
            self._smi = amdsmi
        except Exception as e:  # noqa: BLE001 - a missing reading is reported, not fatal
            self.err = f"amdsmi unavailable: {e}"

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        clk = m.get("current_gfxclk")
        if not isinstance(clk, (int, float)):
            clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
            clk = sum(clks) / len(clks) if clks else None
        pw = m.get("current_socket_power")
        if not isinstance(pw, (int, float)):
            pw = m.get("average_socket_power")
        return clk, pw if isinstance(pw, (int, float)) else None

    def _run(self):
        while not self._stop.is_set():
            try:
                c, p = self._read()
                if c is not None:
                    self.clk.append(c)
                if p is not None:
                    self.pw.append(p)
            except Exception as e:  # noqa: BLE001
                self.err = f"amdsmi read failed: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self._handle is not None:
            self._thr.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thr.is_alive():
            self._thr.join()


def median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2] if xs else None


def sustained(fn, flops: float, seconds: float, peak_tflops: float, runs: int = 3):
    """The README's sustained-clock protocol: 2 s idle, 1 s of back-to-back
    warm-up launches, then `runs` runs of at least `seconds` of back-to-back
    launches, each timed with one event pair around all of its launches; the
    median run is reported with the median GFX clock and socket power
    sampled during the timed runs, and the fraction of the dense peak scaled
    to that clock (TF/s over peak x clock / 2400 MHz), which separates the
    schedule's efficiency from the power cap."""
    import torch
    time.sleep(2.0)
    t_end = time.perf_counter() + 1.0
    n = 0
    while time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per_run = []
    with PowerClockSampler() as smp:
        for _ in range(runs):
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t_end = time.perf_counter() + seconds
            k = 0
            start.record()
            while time.perf_counter() < t_end:
                fn()
                k += 1
                if k % 16 == 0:
                    torch.cuda.synchronize()   # keeps the host within 16 launches of the GPU
            stop.record()
            torch.cuda.synchronize()
            per_run.append((start.elapsed_time(stop) / k, k))
    per_run.sort()
    ms, k = per_run[len(per_run) // 2]
    rec = {"protocol": f"2 s idle, 1 s warm-up, {runs} runs of >= {seconds} s back-to-back, median run",
           "seconds": seconds, "runs": runs, "launches_median_run": k,
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "ms": round(ms, 4),
           "tflops_runs": [round(flops / (m * 1e-3) / 1e12, 2) for m, _ in per_run],
           "gfxclk_mhz": median(smp.clk), "socket_power_w": median(smp.pw), "samples": len(smp.clk)}
    clk = rec["gfxclk_mhz"]
    rec["frac_of_clock_scaled_peak"] = (round(rec["tflops"] / (peak_tflops * clk / 2400.0), 4)
                                        if isinstance(clk, (int, float)) and clk > 0 else None)
    if smp.err:
        rec["note"] = smp.err
    return rec


def settle(fn, seconds: float):
    """Back-to-back launches of fn() for `seconds` (the board leaves its idle
    power state), keeping the host within 16 launches of the GPU."""
    import torch
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_launches(fn, steps, warmup, settle_seconds: float = 0.0):
    """Average milliseconds of fn() over `steps` back-to-back launches,
    bracketed by events on the current stream (the stream fn launches on),
    after `settle_seconds` of back-to-back launches and `warmup` launches."""
    import torch
    if settle_seconds > 0:
        settle(fn, settle_seconds)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    stop = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        start[i].record()
        fn()
        stop[i].record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in zip(start, stop)]
    return sum(ms) / len(ms), ms


CPU_BLOCK_ROWS = 512


def _cpu_worker(job):
    """One worker of the CPU baseline: head slices of the headline workload's
    shape (each its own seeded draw), float64 oracle rows from the last row
    down in blocks, until the deadline; one BLAS thread. Returns rows, head
    slices begun, FLOPs and compute time (input draws excluded)."""
    index, deadline = job
    from threadpoolctl import threadpool_limits
    import numpy as np
    import oracle
    from workloads import WORKLOADS
    w = WORKLOADS[4]
    S, dqk, dv = w.seqlen, w.d_qk, w.d_v
    rows_done, slices, flops, busy = 0, 0, 0.0, 0.0
    with threadpool_limits(limits=1):
        while time.time() < deadline:
            rng = np.random.Generator(np.random.PCG64([w.seed, index, slices]))
            q = oracle.bf16_round(rng.standard_normal((S, dqk), dtype=np.float32))[None, None]
            k = oracle.bf16_round(rng.standard_normal((S, dqk), dtype=np.float32))[None, None]
            v = oracle.bf16_round(rng.standard_normal((S, dv), dtype=np.float32))[None, None]
            slices += 1
            for r1 in range(S, 0, -CPU_BLOCK_ROWS):
                if time.time() >= deadline:
                    break
                rows = np.arange(max(0, r1 - CPU_BLOCK_ROWS), r1)
                t0 = time.perf_counter()
                oracle.causal_attention_rows_ref(q, k, v, 0, 0, rows, layout="bhsd")
                busy += time.perf_counter() - t0
                flops += float(np.sum(rows + 1)) * (dqk + dv) * 2.0
                rows_done += len(rows)
    return rows_done, slices, flops, busy


def cpu_baseline(seconds_budget: float):
    """The float64 oracle on a bounded sample of the headline workload: one
    head slice per worker process (one BLAS thread each, as numpy's
    elementwise exponential runs on one thread), the last query rows first,
    for about seconds_budget of wall time. Run before the GPU is touched;
    workers are fresh interpreters (spawn)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    n = max(1, min(16, os.cpu_count() or 1))
    deadline = time.time() + seconds_budget
    t0 = time.perf_counter()
    # a worker that dies raises here (BrokenProcessPool) instead of hanging
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_cpu_worker, [(i, deadline) for i in range(n)]))
    wall = time.perf_counter() - t0
    rows_done = sum(r[0] for r in res)
    slices = sum(r[1] for r in res)
    # aggregate rate: each worker's FLOPs over its own compute time
    value = sum(r[2] / r[3] for r in res if r[3] > 0) / 1e12
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": value, "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "sample": f"float64 oracle on {rows_done} query rows of {slices} head slices of the bf16 d_qk=192 "
                      f"S=16384 workload's shape ({n} worker processes with one BLAS thread each, last rows first, "
                      f"{CPU_BLOCK_ROWS}-row blocks), {wall:.1f} s wall on {cpu} ({os.cpu_count()} logical CPUs "
                      f"visible); sum over workers of causal FLOPs of their rows / their compute time"}


def range_or_merge_case(name, zy, args):
    """Time one partial-range case (TFLOP/s over visible pairs) or the merge
    (GB/s of its algorithmic bytes against the HBM peak)."""
    import torch
    from workloads import WORKLOADS, generate
    w = WORKLOADS[3]
    dev = torch.device("cuda:0")
    S, H, Hk, d = w.seqlen, w.nheads, w.nheads_k, w.d_qk
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in generate(w))
    if name == MERGE_CASE:
        oa = torch.empty((1, S, H, d), dtype=torch.bfloat16, device=dev)
        la = torch.empty((1, H, S), dtype=torch.float32, device=dev)
        ob, lb = torch.empty_like(oa), torch.empty_like(la)
        # two partial results: keys [0, S/2) and [S/2, S)
        h2 = S // 2
        zy.zyfa_fwd_range(q, k[:, :h2].contiguous(), v[:, :h2].contiguous(), 0, 0, oa, la)
        zy.zyfa_fwd_range(q, k[:, h2:].contiguous(), v[:, h2:].contiguous(), 0, h2, ob, lb)
        out, lse = torch.empty_like(oa), torch.empty_like(la)
        fn = lambda: zy.zyfa_lse_merge(oa, la, ob, lb, out, lse)
        ms, _ = time_launches(fn, args.steps, args.warmup, args.settle_seconds)
        nbytes = 3 * oa.numel() * 2 + 3 * la.numel() * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"gbs": round(gbs, 1), "ms": round(ms, 4), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                "bytes": nbytes, "shape": f"batch 1, seqlen {S}, nheads {H}, d_v {d}, bshd"}
    dtype = RANGE_CASES[name]
    Sq = CHUNK_Q
    qc = q[:, S - Sq:].contiguous()
    out = torch.empty((1, Sq, H, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, H, Sq), dtype=torch.float32, device=dev)
    if dtype == "bf16":
        fn = lambda: zy.zyfa_fwd_range(qc, k, v, S - Sq, 0, out, lse)
    else:
        (q8, qs), (k8, ks), (v8, vs) = (zy.zyfa_fp8_quantize(x) for x in (qc, k, v))
        fn = lambda: zy.zyfa_fwd_range(q8, k8, v8, S - Sq, 0, out, lse, q_descale=qs, k_descale=ks, v_descale=vs)
    fn()
    torch.cuda.synchronize()
    ms, _ = time_launches(fn, args.steps, args.warmup, args.settle_seconds)
    tf = range_flops(1, H, Sq, S, S - Sq, d, d) / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 2), "ms": round(ms, 4), "pct_of_peak": round(100 * tf / PEAK_TFLOPS[dtype], 2),
            "shape": f"{Sq} queries at positions {S - Sq}.. over {S} keys, nheads {H}/{Hk}, d {d}, bshd, LSE"}


def context_setup(name, zy):
    """Inputs and the launch of one README-configuration case: (fn, flops)."""
    import numpy as np
    import torch
    dtype, dqk, S, readme = CONTEXT_CASES[name]
    H = max(32, 262144 // S)
    rng = np.random.Generator(np.random.PCG64(dqk))
    dev = torch.device("cuda:0")
    q, k = (torch.from_numpy(0.1 * rng.standard_normal((1, S, H, dqk), dtype=np.float32)).to(torch.bfloat16).to(dev)
            for _ in range(2))
    v = torch.from_numpy(0.1 * rng.standard_normal((1, S, H, 128), dtype=np.float32)).to(torch.bfloat16).to(dev)
    out = torch.empty((1, S, H, 128), dtype=torch.bfloat16, device=dev)
    if dtype == "bf16":
        fn = lambda: zy.zyfa_fwd(q, k, v, out)
    else:
        (q8, qs), (k8, ks), (v8, vs) = (zy.zyfa_fp8_quantize(x) for x in (q, k, v))
        fn = lambda: zy.zyfa_fwd(q8, k8, v8, out, q_descale=qs, k_descale=ks, v_descale=vs)
    return fn, float(H) * S * S * (dqk + 128)


def protocol_a(zy, runs: int = 3, warmup: int = 500, timed: int = 100, idle: float = 5.0):
    """The README's kernel-benchmark protocol on its own configuration (the
    CONTEXT_CASES): before each case 5 s idle, then 500 warm-up launches and
    the mean of 100 timed back-to-back launches (one event pair); three runs
    with the case order rotated; the median run per case."""
    import torch
    names = list(CONTEXT_CASES)
    setups = {n: context_setup(n, zy) for n in names}
    per = {n: [] for n in names}
    for r in range(runs):
        for n in names[r % len(names):] + names[:r % len(names)]:
            fn, flops = setups[n]
            torch.cuda.synchronize()
            time.sleep(idle)
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            for _ in range(timed):
                fn()
            stop.record()
            torch.cuda.synchronize()
            per[n].append(flops / (start.elapsed_time(stop) / timed * 1e-3) / 1e12)
            print(f"protocol A run {r} {n}: {per[n][-1]:.1f} TF/s", file=sys.stderr, flush=True)
    res = {}
    for n in names:
        t = sorted(per[n])[len(per[n]) // 2]
        readme = CONTEXT_CASES[n][3]
        res[n] = {"tflops": round(t, 2), "runs": [round(x, 1) for x in per[n]], "readme_mi355x_tflops": readme,
                  "ratio_to_readme": round(t / readme, 3)}
    return {"protocol": f"{idle:g} s idle, {warmup} warm-up launches, mean of {timed}, {runs} runs with the order "
                        f"rotated, median run", "cases": res}


def context_case(name, zy, args):
    """The README's benchmark configuration (see CONTEXT_CASES)."""
    import numpy as np
    import torch
    dtype, dqk, S, readme = CONTEXT_CASES[name]
    H = max(32, 262144 // S)
    rng = np.random.Generator(np.random.PCG64(dqk))
    dev = torch.device("cuda:0")
    q, k = (torch.from_numpy(0.1 * rng.standard_normal((1, S, H, dqk), dtype=np.float32)).to(torch.bfloat16).to(dev)
            for _ in range(2))
    v = torch.from_numpy(0.1 * rng.standard_normal((1, S, H, 128), dtype=np.float32)).to(torch.bfloat16).to(dev)
    out = torch.empty((1, S, H, 128), dtype=torch.bfloat16, device=dev)
    if dtype == "bf16":
        fn = lambda: zy.zyfa_fwd(q, k, v, out)
    else:
        (q8, qs), (k8, ks), (v8, vs) = (zy.zyfa_fp8_quantize(x) for x in (q, k, v))
        fn = lambda: zy.zyfa_fwd(q8, k8, v8, out, q_descale=qs, k_descale=ks, v_descale=vs)
    fn()
    torch.cuda.synchronize()
    ms, _ = time_launches(fn, args.steps, args.warmup, args.settle_seconds)
    tf = float(H) * S * S * (dqk + 128) / (ms * 1e-3) / 1e12
    return {"tflops": round(tf, 2), "ms": round(ms, 4), "pct_of_peak": round(100 * tf / PEAK_TFLOPS[dtype], 2),
            "readme_mi355x_tflops": readme, "ratio_to_readme": round(tf / readme, 3),
            "shape": f"MHA, batch 1, seqlen {S}, {H} heads, d_qk {dqk}, d_v 128, bshd, N(0, 0.1^2)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the attention path runs on one GPU and bench.py measures one GPU; run with --gpus 1"}))
        sys.exit(2)
    # the CPU baseline runs first, in fresh worker processes, before this
    # process touches the GPU
    cpu = None if args.no_cpu else cpu_baseline(args.cpu_seconds)
    import numpy as np
    import torch
    import causal_flashattention_prefill_amd as zy
    from workloads import WORKLOADS, generate

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.protocol_a:
        print(json.dumps({"protocol_a": protocol_a(zy)}), flush=True)
        return
    cases = args.only.split(",") if args.only else ALL_CASES
    if args.copy_mib:
        # reference for the byte counters: a device-to-device copy of a
        # source that has been written first
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        src.fill_(0x5A)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res = {}
    sustain = None
    for name in cases:
        if name in CONTEXT_CASES:
            res[name] = context_case(name, zy, args)
            torch.cuda.empty_cache()
            continue
        if name in RANGE_CASES or name == MERGE_CASE:
            res[name] = range_or_merge_case(name, zy, args)
            torch.cuda.empty_cache()
            continue
        wid, dtype = CASES[name]
        w = WORKLOADS[wid].resized(**RESIZED[name]) if name in RESIZED else WORKLOADS[wid]
        q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in generate(w))
        out = torch.empty(w.shape("q")[:-1] + (w.d_v,), dtype=torch.bfloat16, device=dev)
        if dtype == "bf16":
            fn = lambda: zy.zyfa_fwd(q, k, v, out, layout=w.layout)
        else:
            (q8, qs), (k8, ks), (v8, vs) = (zy.zyfa_fp8_quantize(x) for x in (q, k, v))
            pm = PMODE.get(name, "default")
            fn = lambda: zy.zyfa_fwd(q8, k8, v8, out, layout=w.layout, q_descale=qs, k_descale=ks, v_descale=vs,
                                     p_mode=pm)
        # context cases: no quantizer timing, no sustained run
        extra = name in RESIZED or name in PMODE or name in EXTRA
        if dtype == "fp8" and not extra:
            msq, _ = time_launches(lambda: [zy.zyfa_fp8_quantize(x, x8, xs) for x, x8, xs in
                                            ((q, q8, qs), (k, k8, ks), (v, v8, vs))], args.steps, args.warmup,
                                   args.settle_seconds)
            res[name + "_quantize_qkv_ms"] = round(msq, 4)
            # q and k rotated before quantization (same signs), v plain: the
            # README's recipe for models (the 128-point Hadamard rotation);
            # attention then runs unchanged
            signs = np.where(np.random.default_rng(0).random(w.d_qk) < 0.5, -1, 1).astype(np.int8)
        if dtype == "fp8" and not extra and w.d_qk == 128:
            msr, _ = time_launches(lambda: [zy.zyfa_fp8_quantize_rotated(x, signs, x8, xs) for x, x8, xs in
                                            ((q, q8, qs), (k, k8, ks))], args.steps, args.warmup,
                                   args.settle_seconds)
            nb = (q.numel() + k.numel()) * 3      # read bf16 once, write e4m3 once
            res[name + "_rotate_quantize_qk"] = {"ms": round(msr, 4), "gbs": round(nb / (msr * 1e-3) / 1e9, 1),
                                                 "note": "algorithmic bytes (2 B read + 1 B written per element); "
                                                         "the kernels read the input twice"}
            (q8, qs), (k8, ks) = (zy.zyfa_fp8_quantize(x) for x in (q, k))
        fn()
        torch.cuda.synchronize()
        ms, _ = time_launches(fn, args.steps, args.warmup, args.settle_seconds)
        tf = w.flops() / (ms * 1e-3) / 1e12
        tr = stored_traffic(name, dtype)
        res[name] = {"tflops": round(tf, 2), "ms": round(ms, 4),
                     "pct_of_peak": round(100 * tf / PEAK_TFLOPS[dtype], 2),
                     "hbm_traffic_bytes": None if tr is None else int(tr)}
        if args.sustain_seconds > 0 and not extra:
            # every 16K gate case gets the sustained-clock reading; the
            # headline's is also reported at the top level
            res[name]["sustained"] = sustained(fn, w.flops(), args.sustain_seconds, PEAK_TFLOPS[dtype])
            if name == (HEADLINE if HEADLINE in cases else cases[0]):
                sustain = res[name]["sustained"]
        del q, k, v, out
        torch.cuda.empty_cache()

    attn = [c for c in cases if c in CASES]
    if not attn:
        # only partial-range or merge cases were asked for (profiling runs)
        print(json.dumps({"cases": res}), flush=True)
        return
    head = HEADLINE if HEADLINE in res else attn[0]
    tflops, ms = res[head]["tflops"], res[head]["ms"]
    hdt = CASES[head][1]
    line = {
        "metric": "causal prefill attention TFLOP/s (bf16, fp8) at 16K tokens; % of MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": hdt,
        "data": "synthetic",
        "config": {
            "workload": DESCRIPTIONS[head],
            "global_batch": WORKLOADS[CASES[head][0]].batch, "seq_len": WORKLOADS[CASES[head][0]].seqlen,
            "parallelism": "none (1 GPU)",
            "cases": res,
        },
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_TFLOPS[hdt],
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS[hdt], 4),
                     "traffic": res[head]["hbm_traffic_bytes"]},
    }
    if sustain is not None:
        line["sustained"] = sustain
    if not args.no_cpu:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
