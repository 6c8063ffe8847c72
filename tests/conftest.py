"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; all
other tests run on the CPU. The marker is registered here so that
``-m "not gpu"`` and ``-m gpu`` select cleanly.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
