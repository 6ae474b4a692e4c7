import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libhypic")
    config.addinivalue_line("markers", "slow: long CPU reference runs")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _device_status_after_gpu_test(request):
    """After every GPU test: synchronise and fail if a kernel's bounded internal wait gave up
    during the test (its outputs would be unreliable)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    if not torch.cuda.is_available():
        return
    import linear_attention_state_chunked_amd as H
    H.hypic_device_status()
