"""The benchmark's command-line contract on the CPU: more than one GPU is
refused with a message, and the case tables and FLOP counts are consistent."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--no-cpu"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_case_tables():
    assert bench.HEADLINE in bench.CASES
    for name, (wid, dtype) in bench.CASES.items():
        assert wid in WORKLOADS and dtype in bench.PEAK_TFLOPS
        assert name in bench.DESCRIPTIONS
    assert set(bench.RESIZED) <= set(bench.CASES) and set(bench.PMODE) <= set(bench.CASES)
    assert len(set(bench.ALL_CASES)) == len(bench.ALL_CASES)


def test_range_flops_counts_visible_pairs():
    # whole-sequence causal attention: S (S + 1) / 2 visible pairs per head
    S, d = 1000, 128
    assert bench.range_flops(1, 2, S, S, 0, d, d) == 2 * (S * (S + 1) // 2) * 2 * (d + d)
    # a chunk of the last rows over the whole prefix
    Sq, Sk = 10, 50
    pairs = sum(min(Sk, r + (Sk - Sq) + 1) for r in range(Sq))
    assert bench.range_flops(1, 1, Sq, Sk, Sk - Sq, d, d) == pairs * 2 * (d + d)
