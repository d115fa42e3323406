import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (large shards)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(autouse=True)
def _name_gpu_case(request):
    """Name every GPU case (flushed) before it touches the device, and release the
    caching allocator's memory afterwards so large cases do not pile up."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield
    try:
        import torch
        if torch.cuda.is_available():
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
    except Exception:
        pass


@pytest.fixture(scope="session")
def Z():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import zero_partitioned_optimizer_amd as Z
    Z.lib()
    return Z
