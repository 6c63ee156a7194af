import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib(oracle_pool):
    """The built HIP library, loaded through the C-ABI binding; fails loudly if absent.

    Depends on the oracle pool so that its worker processes start before this
    process initialises the GPU."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    from paged_kv_gqa_planner_amd import binding

    binding.load()  # raises if the shared library is missing
    return binding


@pytest.fixture(scope="session")
def oracle_pool():
    """Worker processes running the oracle over (request, KV head) items."""
    from tests.oracle_pool import OraclePool

    with OraclePool() as pool:
        yield pool
