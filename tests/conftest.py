"""Shared pytest set-up.

Markers: ``gpu`` tests need an MI355X and call the HIP library through its C
ABI; everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU-side work (full-size workloads)")


def gpu_available() -> bool:
    # device_count() does not initialise the HIP runtime in this process, so
    # a test may still start child processes afterwards.
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover - torch import failure means no GPU path
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no ROCm GPU visible (gpu tests run on an MI355X)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
