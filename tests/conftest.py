import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "device_library: calls entry points that only the full HIP library exports")
    # A host-only build of the library (the sanitizer run of the CPU tests)
    # replaces the HIP library for the whole session.
    host_lib = os.environ.get("PKV_HOST_LIBRARY")
    if host_lib:
        import paged_kv_decode_step_amd as pkv
        pkv.load_library(host_lib, host_only=True)


def pytest_collection_modifyitems(config, items):
    if not os.environ.get("PKV_HOST_LIBRARY"):
        return
    skip = pytest.mark.skip(reason="the host-only library does not export this entry point")
    for item in items:
        if "device_library" in item.keywords:
            item.add_marker(skip)
