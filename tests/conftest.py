import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large workload, runs for tens of seconds")


@pytest.fixture(scope="session", autouse=True)
def _built_host_libs():
    """The generator and the oracle are plain C; build them once if missing."""
    import gen
    import oracle
    if not os.path.exists(os.path.join(ROOT, "gen", "libgsagen.so")):
        gen.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()
    yield
