import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0.  Fails loudly (no fallback) when the
    library is missing; skips only when the machine has no GPU at all."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    import bounded_generation_slm_amd as slm
    return slm.Context(device=0)
