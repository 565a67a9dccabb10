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
