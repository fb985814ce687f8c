import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size CPU cases (tens of seconds)")
    config.addinivalue_line("markers", "host_pointers: passes host pointers to entry points that can launch "
                                       "kernels (argument-check tests); skipped where a GPU is visible")


def _gpu_visible():
    """True when a GPU is visible to this process.  torch's device count does
    not initialise the HIP runtime."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    # Argument-check tests hand host buffers to entry points that launch
    # kernels once their checks pass; they rely on every check returning
    # first.  Where a GPU is visible a regressed check would launch a kernel
    # on pageable host memory, so those tests run on CPU-only machines only.
    if not any(item.get_closest_marker("host_pointers") for item in items):
        return
    if not _gpu_visible():
        return
    skip = pytest.mark.skip(reason="passes host pointers to launching entry points; CPU-only machines run it")
    for item in items:
        if item.get_closest_marker("host_pointers"):
            item.add_marker(skip)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture
def golden():
    return load_golden
