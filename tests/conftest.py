import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    # GPU tests last, so a CPU-only failure shows up before any GPU work.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


@pytest.fixture(scope="session")
def libuq():
    """The built library (built once here if nothing is built yet)."""
    import decode_attention_bit_amd as uq
    if not os.path.exists(uq.library_path()):
        from decode_attention_bit_amd import build
        build.build()
    return uq._load()
