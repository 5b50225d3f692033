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
def params():
    from manifold_constrained_hyper_mhc_amd.synthetic import Params
    return Params()


@pytest.fixture(autouse=True)
def _name_gpu_case(request):
    # name the case before any GPU work, so a run that ends abruptly says which
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
