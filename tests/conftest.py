import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large synthetic workloads")


@pytest.fixture(scope="session", autouse=True)
def _build_c_helpers():
    """The plain-C generator and oracle build in a second with gcc."""
    import oracle
    import synth
    synth.build()
    oracle.build()
