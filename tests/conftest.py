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
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "_bitlinear_build", os.path.join(ROOT, "ternary_weight_absmean_amd", "_build.py"))
    build_mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build_mod)
    if not os.path.exists(build_mod.LIB_PATH):
        build_mod.build()
    yield
