import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU statistics test")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is present; returns the loaded HIP binding."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import draft_verification_vocab_amd as sv
    sv.require_library()
    return sv


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on stderr before it runs, so a failure that takes the
    process down still says which case was running."""
    if request.node.get_closest_marker("gpu"):
        sys.__stderr__.write(f"[gpu-case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
