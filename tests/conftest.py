import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU case")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded C-ABI library, for GPU tests. Fails loudly when missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a GPU")
    import fp4_quantized_diffusion_amd as fq
    fq.load_library()
    return fq
