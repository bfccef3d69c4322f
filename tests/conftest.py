import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI)")


@pytest.fixture(scope="session")
def ref():
    """The CPU oracle (built on first use)."""
    from oracle import fwref
    fwref.lib()
    return fwref
