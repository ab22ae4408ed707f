import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmc2")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to minutes)")


@pytest.fixture(scope="session", autouse=True)
def _built_host_libs():
    """The generator and the oracle are plain C built with gcc; build them once if absent."""
    import mc2_inputs
    import oracle
    mc2_inputs.build(force=False)
    oracle.build(force=False)
    yield
