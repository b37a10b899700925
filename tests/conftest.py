import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")
    config.addinivalue_line("markers", "slow: full-size parity case")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def gpu():
    """The binding, after checking that a GPU is present and the library loads."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import compressed_kv_cache_decode_amd as csa2
    csa2.lib()  # raises if libcsa2.so is missing
    return csa2
