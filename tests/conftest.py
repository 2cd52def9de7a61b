import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are selected with -m gpu on a GPU machine.  Without a device they
    # are skipped rather than run against any fallback (there is none).
    if any("gpu" in item.keywords for item in items):
        import torch
        if not torch.cuda.is_available():
            skip = pytest.mark.skip(reason="no GPU visible")
            for item in items:
                if "gpu" in item.keywords:
                    item.add_marker(skip)
