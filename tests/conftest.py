import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_required(request):
    """GPU tests fail (never skip) when no GPU is visible: the HIP path must run."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("test marked gpu but no HIP device is visible")
        print(f"\n[gpu] {request.node.nodeid}", flush=True)
    yield
