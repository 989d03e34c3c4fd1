"""Mutation check of the oracle's pins (CPU only).

The oracle is trusted because its pins (tests/test_oracle_*.py) tie it to
what the pages and the mathematics fix. That holds only if a plausible
mistake anywhere in it fails a pin. tests/oracle_mutants.py plants one
mistake at a time (a mask off by one, no mask, a transposed operand, a
dropped normalisation or max, LSE in the wrong base, a wrong GQA map, scale
or layout axis, a merge that keeps the larger LSE or swaps its weights, a
wrong e4m3 bias or tie rule, bf16 truncation, a descale rounded down or
without its 2^-126 floor, rotation signs on the wrong axis or no 1/sqrt(d),
a key mean over the wrong axis); each is run against the pins in a child
pytest process, which must fail. A control run without a mutant must pass.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = ["test_oracle_attention.py", "test_oracle_partial.py", "test_oracle_codecs.py",
        "test_oracle_quantize.py", "test_oracle_rotation.py"]


def _run(mutant):
    env = dict(os.environ, ZYFA_ORACLE_MUTANT=mutant, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    if not mutant:
        env.pop("ZYFA_ORACLE_MUTANT")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join(HERE, f) for f in PINS]],
                       env=env, cwd=os.path.dirname(HERE), capture_output=True, text=True, timeout=600)
    last = [l for l in r.stdout.splitlines() if l.strip()][-1:] or [r.stderr[-300:]]
    return mutant, r.returncode, last[0]


def test_every_planted_mistake_fails_a_pin():
    names = [""] + sorted(MUTANTS)
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        res = {m: (rc, last) for m, rc, last in ex.map(_run, names)}
    rc0, last0 = res.pop("")
    assert rc0 == 0, f"the pins fail without a mutant: {last0}"
    # exit status 1: tests ran and at least one failed (2 and above would be
    # a crash of the run itself, which proves nothing about the pins)
    survivors = {m: last for m, (rc, last) in res.items() if rc == 0}
    broken = {m: (rc, last) for m, (rc, last) in res.items() if rc not in (0, 1)}
    assert not broken, f"mutant runs that did not complete: {broken}"
    assert not survivors, f"planted mistakes that every pin passes: {survivors}"
