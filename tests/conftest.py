import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libwkv")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host time for the oracle)")


def _gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover - torch import failure
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible: gpu-marked tests run on an MI355X box")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
