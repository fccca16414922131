import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; GPU tests fail (not skip) when it is missing."""
    import torch

    from parallax_local_linear_plx_amd import binding

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    return binding.lib()
