import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of host-side input generation)")


@pytest.fixture(scope="session")
def qsa_lib():
    """The built HIP library (built first only if it is missing)."""
    from block_sparse_attention_37_amd import qsa
    import os as _os
    if not _os.path.exists(qsa.LIB_PATH):
        from block_sparse_attention_37_amd import build
        build.build()
    return qsa.lib()


@pytest.fixture(scope="session")
def gpu(qsa_lib):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")
