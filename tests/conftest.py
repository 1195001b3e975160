import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs; minutes of CPU work")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on cuda:0; the GPU tests fail loudly if it cannot load."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import paged_kv_cache_69_amd as pa

    pa.load_library()
    return pa
