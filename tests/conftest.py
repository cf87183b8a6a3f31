import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def _ensure_built():
    lib = os.path.join(ROOT, "sparse_attention_decode_lightning_amd", "libdsa.so")
    if not os.path.exists(lib):
        from sparse_attention_decode_lightning_amd import build as _b
        _b.build(verbose=False)


_ensure_built()
