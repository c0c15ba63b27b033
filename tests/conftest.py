import os
import sys

import pytest

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded; the GPU tests fail (not skip) when it is absent."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import head_exchange_amd as hx
    hx.load()          # raises when the extension is not built
    return hx
