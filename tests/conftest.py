import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) only when no GPU exists at all; on a GPU
    # machine a missing or broken library makes them fail loudly.
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


class _Knobs:
    """Sets the library's tuning knobs (the ADDRMS_* names of addrms.h) for
    one test and restores them afterwards."""

    def __init__(self):
        self.prev = {}

    def setenv(self, name: str, value):
        import add_rmsnorm_amd as ar
        prev = ar.set_knob(name, int(value))
        self.prev.setdefault(name, prev)

    def restore(self):
        import add_rmsnorm_amd as ar
        for name, v in self.prev.items():
            ar.set_knob(name, v)
        self.prev.clear()


@pytest.fixture
def knobs():
    k = _Knobs()
    yield k
    k.restore()
