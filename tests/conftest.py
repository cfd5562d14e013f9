import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def pkv_lib():
    """The built HIP library (built once if it is absent)."""
    import paged_kv_cache_281_amd as pkv
    if not os.path.exists(pkv.library_path()):
        from paged_kv_cache_281_amd import build
        build.build()
    pkv.load()
    return pkv
