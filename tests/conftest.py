import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _flush_name(item):
    # Name the case before it touches the GPU, so a crash still says which case ran.
    sys.stdout.write(f"\n[case] {item.nodeid}\n")
    sys.stdout.flush()


def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu") is not None:
        _flush_name(item)


def pytest_terminal_summary(terminalreporter):
    """The largest rel-L2 against the fp64 oracle per test family, quantity and
    input dtype over the tests that ran (GPU runs only)."""
    try:
        from gpu_helpers import MAXIMA
    except ImportError:
        return
    if not MAXIMA:
        return
    tr = terminalreporter
    tr.write_sep("-", "largest rel-L2 against the oracle (family / quantity / inputs)")
    for (fam, name, dtype), e in sorted(MAXIMA.items()):
        tr.write_line(f"{fam:52s} {name:20s} {dtype:5s} {e:.2e}")
