"""Build the gfx950 shared library libzyfa.so in place with hipcc.

Usage: python -m causal_flashattention_prefill_amd.build  (or build()).
Always recompiles; the library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzyfa.so")

SOURCES = ["api.cpp", "args.cpp", "plan.cpp", "attn_bf16.hip", "attn_fp8.hip", "fp8_quantize.hip", "lse_merge.hip", "noalloc.hip"]
# Extra flags per source. The attention kernels never see NaN scores, so
# max/min need no NaN quieting (IEEE mode off): without this every fmaxf of
# a matrix-instruction result costs an extra canonicalising instruction.
EXTRA_FLAGS = {
    "attn_fp8.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
    "attn_bf16.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
}
BUILD_DIR = os.path.join(HERE, "_build")
# The MFMA-shape microbenchmark (bench_mfma_shapes.py): its own library, not
# part of the attention library.
MB_SOURCE = "mfma_shapes.hip"
MB_LIB = os.path.join(HERE, "libzyfa_mfma_shapes.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions (v_pk_*_f32) are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-Wno-inline-asm",  # m0 is clobbered on purpose by the direct-to-LDS load asm
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else (shutil.which("hipcc") or "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        cmd = [hipcc(), *compile_flags, *EXTRA_FLAGS.get(src, []), *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, _run(cmd, verbose)))
    failed = []
    for src, p in jobs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed to compile " + ", ".join(failed))
    tmp = LIB + ".tmp"
    p = _run([hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp], verbose)
    out, _ = p.communicate()
    if p.returncode != 0:
        sys.stderr.write(out)
        raise RuntimeError("hipcc failed to link libzyfa.so")
    os.replace(tmp, LIB)
    tmp = MB_LIB + ".tmp"
    p = _run([hipcc(), *HIPCC_FLAGS, os.path.join(CSRC, MB_SOURCE), "-o", tmp], verbose)
    out, _ = p.communicate()
    if p.returncode != 0:
        sys.stderr.write(out)
        raise RuntimeError("hipcc failed to build the MFMA-shape microbenchmark")
    os.replace(tmp, MB_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
