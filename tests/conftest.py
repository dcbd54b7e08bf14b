import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP path's binding where a GPU is present; the test fails loudly when the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from resident_rl_rollout_amd import binding
    return binding.lib()
