import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than ~30 s")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded once; the GPU tests fail loudly if it is missing."""
    import torch
    from gpt_transformer_step_train_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return binding.load()
