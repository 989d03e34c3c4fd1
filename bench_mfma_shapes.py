"""Equal-FLOP matrix-instruction streams of two tile shapes on one MI355X, at
the board's power cap: the measurement behind the attention kernels' MFMA
shape ("Attention at the Power Cap", sections 2 and 3.2, compares
16x16x32 and 32x32x16 bf16 streams by TF/s, clock and power at the cap),
and the rate of the older v_mfma_f32_16x16x32_fp8_fp8, which the FP8 kernel
uses for the channels past 128 of d_qk = 192 (cycles per instruction =
FLOP per instruction x 1024 SIMDs x clock / FLOP/s).

Each case runs the microbenchmark kernels of csrc/mfma_shapes.hip (one
512-thread workgroup per CU, 8 waves, independent instructions on random
operands) back to back with bench.py's sustained-clock protocol: 2 s idle,
1 s warm-up, three runs of >= --seconds, the median run, with the median
GFX clock and socket power. The shapes are interleaved (A B A B) so drift
in the board's temperature falls on both.

    python bench_mfma_shapes.py [--seconds 3] [--rounds 2]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

KINDS = {0: ("bf16", "v_mfma_f32_16x16x32_bf16"), 1: ("bf16", "v_mfma_f32_32x32x16_bf16"),
         2: ("fp8", "v_mfma_scale_f32_16x16x128_f8f6f4"), 3: ("fp8", "v_mfma_scale_f32_32x32x64_f8f6f4"),
         4: ("fp8", "v_mfma_f32_16x16x32_fp8_fp8")}
ITERS = {0: 2000, 1: 2000, 2: 1000, 3: 1000, 4: 1000}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seconds", type=float, default=3.0)
    ap.add_argument("--rounds", type=int, default=2)
    args = ap.parse_args()
    import torch
    from bench import PEAK_TFLOPS, sustained
    from causal_flashattention_prefill_amd.build import MB_LIB
    if not os.path.exists(MB_LIB):
        raise RuntimeError(f"{MB_LIB} not built; run causal_flashattention_prefill_amd.build.build()")
    L = ctypes.CDLL(MB_LIB)
    L.mfma_shapes_flop_per_wave_iter.restype = ctypes.c_longlong
    L.mfma_shapes_in_words.restype = ctypes.c_longlong
    L.mfma_shapes_out_floats.restype = ctypes.c_longlong
    L.mfma_shapes_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    dev = torch.device("cuda:0")
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator(device=dev).manual_seed(0)
    nw = L.mfma_shapes_in_words(grid)
    # valid operands: bf16 N(0,1) values, and e4m3fn N(0,1) codes (no NaN codes)
    ins = {"bf16": torch.randn(2 * nw, generator=g, device=dev).to(torch.bfloat16).view(torch.int32),
           "fp8": torch.randn(4 * nw, generator=g, device=dev).to(torch.float8_e4m3fn).view(torch.int32)}
    out = torch.empty(L.mfma_shapes_out_floats(grid), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    res = {k: [] for k in KINDS}
    for r in range(args.rounds):
        for kind in KINDS:
            dt, name = KINDS[kind]
            x = ins[dt]
            flops = float(grid) * 8 * ITERS[kind] * L.mfma_shapes_flop_per_wave_iter(kind)

            def fn(kind=kind, x=x):
                if L.mfma_shapes_launch(kind, x.data_ptr(), out.data_ptr(), ITERS[kind], grid, stream) != 0:
                    raise RuntimeError("launch failed")
            rec = sustained(fn, flops, args.seconds, PEAK_TFLOPS[dt])
            rec["instruction"] = name
            res[kind].append(rec)
            print(f"round {r} {name}: {rec['tflops']} TF/s at {rec['gfxclk_mhz']} MHz, {rec['socket_power_w']} W",
                  file=sys.stderr, flush=True)
    summary = {}
    for kind, recs in res.items():
        dt, name = KINDS[kind]
        best = sorted(recs, key=lambda x: x["tflops"])[len(recs) // 2]
        summary[name] = {"dtype": dt, "tflops_rounds": [x["tflops"] for x in recs],
                         "gfxclk_mhz_rounds": [x["gfxclk_mhz"] for x in recs],
                         "socket_power_w_rounds": [x["socket_power_w"] for x in recs],
                         "tflops": best["tflops"], "gfxclk_mhz": best["gfxclk_mhz"],
                         "socket_power_w": best["socket_power_w"],
                         "frac_of_clock_scaled_peak": best["frac_of_clock_scaled_peak"]}
    print(json.dumps({"mfma_shapes": summary, "grid": grid, "waves_per_cu": 8,
                      "protocol": res[0][0]["protocol"]}), flush=True)


if __name__ == "__main__":
    main()
