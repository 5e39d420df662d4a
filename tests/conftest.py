import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    """The oracle as built in-tree (built here if it is missing)."""
    from oracle import oracle as o
    from oracle import _build
    if not o.LIBRARY.exists():
        _build.build()
    return o.default()
