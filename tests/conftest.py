import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden():
    import json

    with open(os.path.join(ROOT, "tests", "golden", "worked_examples.json")) as f:
        return json.load(f)


@pytest.fixture(autouse=True)
def _device_waits_completed(request):
    """After every GPU test: no bounded device-side wait of the library gave up
    (sf_workspace_check on every workspace the binding created)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    from bit_decode_selective_amd import binding

    if binding._lib is not None:
        binding.check_workspaces()
