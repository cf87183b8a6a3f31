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
        # load the build script by path: importing the package needs the library
        import importlib.util

        path = os.path.join(ROOT, "sparse_attention_decode_lightning_amd", "build.py")
        spec = importlib.util.spec_from_file_location("_dsa_build", path)
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build(verbose=False)


_ensure_built()
