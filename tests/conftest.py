import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def _keep_freed_heap_memory():
    """The oracle allocates and frees score blocks of hundreds of MiB; keep
    freed memory in the process instead of unmapping it, so the next block
    does not page-fault all over again (glibc mallopt: mmap and trim
    thresholds)."""
    try:
        import ctypes

        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-3, 1 << 30)       # M_MMAP_THRESHOLD
        libc.mallopt(-1, (1 << 31) - 1)  # M_TRIM_THRESHOLD
    except (OSError, AttributeError):
        pass


_keep_freed_heap_memory()


def pytest_configure(config):
    import gpu_util

    gpu_util.PYTEST_CONFIG = config
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: multi-minute GPU case (full-size workloads)")


def pytest_collection_modifyitems(config, items):
    # cheap tests first, then the full-size GPU cases, then the test_zz_*
    # files, which must also pass after everything else has run
    def rank(it):
        if os.path.basename(str(it.fspath)).startswith("test_zz_"):
            return 2
        return 1 if it.get_closest_marker("slow") else 0

    items.sort(key=rank)

