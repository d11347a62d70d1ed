"""Test configuration: the `gpu` marker and import paths.

CPU tests (`-m "not gpu"`) cover the oracle against its pins, the host-side
logic and the library's exported symbols; `-m gpu` tests compare the HIP path
with the oracle through the C ABI.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built libwc.so")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Rebuild the CPU oracle when its source is newer than the library."""
    import oracle
    src = os.path.join(ROOT, "oracle", "wc_oracle.c")
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
        oracle.build()
    yield
