import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI on the GPU)")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Build the CPU oracle once per session if it is missing (test infrastructure)."""
    from oracle import build as obuild
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        obuild.build()
    yield
