import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size GPU parity case")


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP library binding; fails loudly when it cannot run."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda is not available")
    import attention_flash_sdpa_amd as fa
    fa.load()   # raises if the shared library is missing
    return fa
