import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size cases (several seconds of oracle time)")


def pytest_collection_modifyitems(config, items):
    # A GPU test that lands on a machine without a GPU is skipped loudly, never
    # silently passed; the driver selects them with -m gpu on the GPU machine.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="NO GPU PRESENT: GPU test not run")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
