import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # GPU tests end the collection order so a CPU failure never hides behind them.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_libs():
    import oracle
    import synth
    if not os.path.exists(oracle._LIB):
        oracle.build(force=True)
    if not os.path.exists(synth._LIB):
        synth.build(force=True)
    yield
