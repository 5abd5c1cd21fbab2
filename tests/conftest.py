import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def splash():
    """The ctypes binding over libsplash_attn.so, built first if it is missing."""
    import layout_agnostic_latent_amd as m
    if not os.path.exists(m.LIB_PATH):
        from layout_agnostic_latent_amd import build as b
        b.build_library()
    return m
