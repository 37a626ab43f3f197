import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def pytest_collection_modifyitems(config, items):
    # Heavier GPU cases run after the small ones so a failure shows up early;
    # the allocation-free entry point's test (test_zz_*) runs last of all.
    items.sort(key=lambda it: 2 if "test_zz_" in it.nodeid else (1 if it.get_closest_marker("slow") else 0))
