import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    # a planted oracle mistake, for the mutation check of the oracle's pins
    # (tests/test_oracle_mutants.py runs the pins in a child process with it)
    mutant = os.environ.get("ZYFA_ORACLE_MUTANT")
    if mutant:
        import oracle_mutants
        oracle_mutants.apply(mutant)
