import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def _ensure_built():
    """Build libgemm.so (and the oracle) in-tree if absent, so a fresh checkout can test."""
    lib = os.path.join(ROOT, "gemm_f32_amd", "libgemm.so")
    if not os.path.exists(lib):
        from gemm_f32_amd import build as _b
        _b.build()


def pytest_sessionstart(session):
    _ensure_built()
