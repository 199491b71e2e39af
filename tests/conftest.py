import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session", autouse=True)
def _synth_built():
    """The seeded input generator is plain C; build it if it is missing."""
    from host_memory_streamed_amd import build
    if not os.path.exists(os.path.join(build.HERE, "libmtsynth.so")):
        build.build_synth()
