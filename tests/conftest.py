import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) through the C ABI")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_required(request):
    """GPU tests fail loudly (never skip) when no HIP device is visible."""
    if request.node.get_closest_marker("gpu") is not None:
        import torch
        if not torch.cuda.is_available():
            pytest.fail("test marked gpu but no HIP device is visible")
    yield
