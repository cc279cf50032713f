import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture
def attn_options():
    """Set process-wide planner switches of the library (attn_set_option) for one
    test; every switch it touched is restored afterwards."""
    import tiled_prefill_amd as tpa

    saved = {}

    def setter(name, value):
        if name not in saved:
            saved[name] = tpa.get_option(name)
        tpa.set_option(name, int(value))

    yield setter
    for name, value in saved.items():
        tpa.set_option(name, value)
