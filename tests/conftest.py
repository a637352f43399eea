import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    gpu_items = [it for it in items if "gpu" in it.keywords]
    if not gpu_items:
        return
    markexpr = (config.getoption("-m") or "").replace(" ", "")
    if markexpr == "gpu":
        # An explicit GPU run must fail loudly when no device is there, never skip.
        return
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if not have_gpu:
        skip = pytest.mark.skip(reason="no GPU visible")
        for item in gpu_items:
            item.add_marker(skip)
