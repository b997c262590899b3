import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle run")


def pytest_collection_modifyitems(config, items):
    # GPU tests print their case before they touch the device, so a fault names it.
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(pytest.mark.usefixtures("_announce_gpu_case"))


@pytest.fixture
def _announce_gpu_case(request):
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
