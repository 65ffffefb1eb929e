import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built libgbreduce")
    config.addinivalue_line(
        "markers", "exhaustive: sweeps all 2^32 float32 bit patterns (skip with GB_EXHAUSTIVE=0)")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("GB_EXHAUSTIVE") != "0":
        return
    skip = pytest.mark.skip(reason="full 2^32 sweep skipped: GB_EXHAUSTIVE=0")
    for item in items:
        if "exhaustive" in item.keywords:
            item.add_marker(skip)
