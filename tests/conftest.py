import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: multi-minute GPU case (full-size workloads)")


def pytest_collection_modifyitems(config, items):
    # run cheap tests first, the full-size GPU cases last
    items.sort(key=lambda it: 1 if it.get_closest_marker("slow") else 0)
