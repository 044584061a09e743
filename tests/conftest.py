import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def built_lib():
    """Path of libmla355.so; built here only if no build exists yet."""
    from latent_kv_attention_amd import build as _build
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    return _build.LIB_PATH
