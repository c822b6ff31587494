import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity cases")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    oracle.build(force=False)
    yield


@pytest.fixture(scope="session")
def crkv_lib():
    """The HIP library, built in-tree if no build is present."""
    import attention_precomputed_chunk_amd as crkv
    from attention_precomputed_chunk_amd import build as crkv_build
    if not os.path.exists(crkv.LIB_PATH):
        crkv_build.build()
    return crkv.lib()
