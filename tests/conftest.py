import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests on a machine without a GPU are skipped with a reason rather
    # than silently passing; on a GPU machine they run and must find the
    # built library (the binding raises if it is missing).
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def _keep_freed_memory_in_heap():
    """Large numpy temporaries are otherwise mmap'ed and unmapped on every
    allocation; on hosts where first-touch page faults are slow that dominates
    the oracle's run time.  Keep freed memory in the heap for reuse."""
    try:
        import ctypes
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-3, 1 << 30)                  # M_MMAP_THRESHOLD
        libc.mallopt(-1, ctypes.c_int(2 ** 31 - 1))  # M_TRIM_THRESHOLD
    except Exception:  # pragma: no cover
        pass


_keep_freed_memory_in_heap()
