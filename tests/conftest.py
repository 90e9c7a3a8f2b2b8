"""Shared pytest set-up: the `gpu` marker, import paths and lazy builds."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C ABI")


@pytest.fixture(scope="session")
def oracle_lib():
    """The fp64 oracle, compiled on first use if it is not built yet."""
    import oracle

    if not os.path.exists(oracle.library_path()):
        oracle.build(force=True)
    return oracle
