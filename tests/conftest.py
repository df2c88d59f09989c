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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    if not os.path.exists(os.path.join(ROOT, "oracle", "libnvfp4_ref.so")):
        oracle.build()
    return oracle


@pytest.fixture(scope="module")
def nv():
    """The GPU library's binding (imports only when a GPU test asks for it)."""
    from block_scale_search_amd import nvfp4
    return nvfp4
