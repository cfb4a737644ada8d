import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


_CAPMAN = None


def progress(msg: str):
    """A progress line that reaches the terminal (or the file it is
    redirected to) at once, also while pytest captures the test's output:
    a GPU case is named before its GPU work starts."""
    if _CAPMAN is not None:
        with _CAPMAN.global_and_fixture_disabled():
            sys.stderr.write(msg + "\n")
            sys.stderr.flush()
    else:
        sys.__stderr__.write(msg + "\n")
        sys.__stderr__.flush()


def pytest_configure(config):
    global _CAPMAN
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    _CAPMAN = config.pluginmanager.getplugin("capturemanager")


def pytest_runtest_setup(item):
    if item.get_closest_marker("gpu"):
        progress(f"[gpu] start {item.nodeid}")


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
