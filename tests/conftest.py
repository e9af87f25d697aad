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


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU test on the real stderr before it runs, so a run that
    dies mid-test still says which case it was in."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
