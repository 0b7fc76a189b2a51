import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when the GPU or the library is missing;
    # they are selected with -m gpu and deselected with -m "not gpu".
    pass


@pytest.fixture(autouse=True)
def _device_status_checks(request):
    """GPU tests run with the binding's device checks on: every library call
    synchronises and fails if its workspace status word reports that a
    bounded in-kernel wait ran out."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import gated_linear_attention_chunked_amd as lam

    lam.set_device_checks(True)
    yield


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.build(force=False)
    return oracle
