import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of CPU time")


def pytest_collection_modifyitems(config, items):
    # GPU tests print what they run (seed, shape, entry point) before each GPU step.
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(pytest.mark.usefixtures("_gpu_announce"))


@pytest.fixture
def _gpu_announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", flush=True)
    yield
