import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device) to run")


@pytest.fixture(scope="session")
def lib():
    """The built libfwt.so (built here if nothing is built yet)."""
    import quantum_state_encoding_amd as qse
    from quantum_state_encoding_amd import build as libbuild
    if not os.path.exists(qse.library_path()):
        libbuild.build()
    return qse.load_library()
