"""Shared pytest setup: markers, import path, and the built library.

Tests marked ``gpu`` need an MI-series GPU and the built HIP library; all
others run on the CPU.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes on the CPU side)")


@pytest.fixture(scope="session")
def built_library():
    """Path of libpa.so, building it once if nothing is built yet."""
    from paged_kv_cache_303_amd import build as pa_build
    path = pa_build.library_path()
    if not os.path.exists(path):
        pa_build.build()
    return path


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is visible; returns the torch device."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda", 0)
