import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload on the GPU")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP path, loaded through its Python binding; fails loudly if the
    built library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_236_amd as pk
    return pk
