import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; GPU tests fail (not skip)
    when it is missing, so a silent fallback can never pass them."""
    import torch
    import sparse_activation_amd as qs
    assert torch.cuda.is_available(), "GPU test collected on a host without a GPU"
    qs.load()
    return qs
