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
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of CPU oracle time)")


@pytest.fixture(scope="session", autouse=True)
def _built_libraries():
    """Build the CPU libraries (and the HIP library) only where nothing is built."""
    import datagen
    import oracle

    datagen.build()
    oracle.build()
    try:
        from ternary_weight_absmean_amd import _build
    except ImportError:
        _build = None
    if _build is not None and not os.path.exists(_build.LIB_PATH):
        _build.build()
    yield
