import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large full-size case")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0; fails loudly if the GPU or the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    from decode_attention_learned_amd import lib

    lib.load()
    return torch.device("cuda:0")
