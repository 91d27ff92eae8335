import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")


def _built():
    return all(os.path.exists(os.path.join(ROOT, p)) for p in (
        "oracle/liboracle.so", "moe_activation_bit_amd/libsynth.so", "moe_activation_bit_amd/libtk.so"))


@pytest.fixture(scope="session", autouse=True)
def _native_libraries():
    # build only when nothing is built; after a source change run build() first
    if not _built():
        import __graft_entry__
        __graft_entry__.build()
    yield
