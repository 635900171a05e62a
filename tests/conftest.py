import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_libraries():
    """Tests load what is built; build only what is missing (CPU only)."""
    from gemm_autotuning_amd import build as b
    from oracle import build_oracle
    if not os.path.exists(b.LIB):
        b.build()
    build_oracle.build(force=False)
    yield
