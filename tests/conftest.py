import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0.  A GPU test never falls back to anything else:
    if the device is there but the library is not, the test errors out."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import reduction_rmsnorm_fwd_amd as fo
    fo.load()  # raises if libfo.so is missing or the device is not gfx950
    return fo
