import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (large inputs, tens of seconds)")


@pytest.fixture(scope="session")
def rf():
    """The HIP library binding. A missing library is an error, never a skip."""
    import cascaded_reductions_amd as rf_mod
    rf_mod.load()  # raises if librf.so is absent or cannot be loaded
    return rf_mod
