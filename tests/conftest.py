import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (seconds to minutes)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on cuda:0; a GPU test fails loudly if either is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import invariant_gemm_token_amd as tig
    tig.load()  # raises if libtig.so is missing or does not load
    return tig
