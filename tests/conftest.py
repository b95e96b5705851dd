import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity through the C-ABI")


@pytest.fixture(scope="session", autouse=True)
def _built_oracle():
    """The oracle is plain C; build it if it is missing (cheap, CPU only)."""
    from oracle import build as ob
    if not os.path.exists(ob.LIB):
        ob.build()
