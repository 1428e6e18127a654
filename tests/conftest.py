import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def _have_gfx950() -> bool:
    try:
        import torch
        if not torch.cuda.is_available():
            return False
        arch = torch.cuda.get_device_properties(0).gcnArchName
        return arch.split(":")[0] == "gfx950"
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # GPU tests are gated on the device architecture, not on whether a library loads:
    # on a gfx950 box a missing library is a failure, not a skip.
    if _have_gfx950():
        return
    skip = pytest.mark.skip(reason="needs a gfx950 GPU")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
