import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def prefill_case():
    """The 256-expert prefill workload's inputs (about 6 GB of weights), drawn
    once per session for the tests that check it at full size."""
    from gemm_mxfp4_dequant_amd import inputs
    return inputs.workload_case(5)
