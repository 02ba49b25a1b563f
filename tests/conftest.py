import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU)")


_ERR_FD = None


def pytest_sessionstart(session):
    # a copy of stderr taken before pytest's output capture starts
    global _ERR_FD
    _ERR_FD = os.dup(2)


def pytest_runtest_setup(item):
    """Name each GPU test on stderr, unbuffered, before it launches anything:
    if a kernel takes the device down, the last line printed names the case."""
    if _ERR_FD is not None and item.get_closest_marker("gpu") is not None:
        os.write(_ERR_FD, f"[gpu test] {item.nodeid}\n".encode())
