import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "device_abi: calls a device entry point's host-side checks (needs the "
                                       "full library, not the host-only sanitizer build)")


def pytest_collection_modifyitems(config, items):
    """Under TDP_LIBRARY's host-only build the device entry points are absent:
    skip the tests that call them (their host checks run in the full build)."""
    if not os.environ.get("TDP_LIBRARY"):
        return
    import overlap_tiling_trapezoidal_amd as tdp
    tdp.load_library()
    if not tdp.HOST_ONLY:
        return
    skip = pytest.mark.skip(reason="host-only library build (TDP_LIBRARY): no device entry points")
    for item in items:
        if "device_abi" in item.keywords or "gpu" in item.keywords:
            item.add_marker(skip)


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
