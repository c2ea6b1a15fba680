import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def gdn_lib():
    """The built libgdn binding; GPU tests fail loudly if it is missing."""
    import torch
    from linear_attention_recurrence_deltanet_amd import gdn
    if not torch.cuda.is_available():
        pytest.fail("gpu test collected without a GPU")
    gdn.load()
    return gdn
