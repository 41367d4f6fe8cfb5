import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the HIP library")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of CPU oracle work")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a GPU; fails loudly (never skips to a CPU path) when absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test run without a visible GPU")
    import kv_reuse_amd
    kv_reuse_amd.load()
    return kv_reuse_amd
