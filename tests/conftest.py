import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(TESTS, "golden")


class TuningEnv:
    """RR_* tuning variables set for one test.  The library reads them once
    per process, so every change is followed by rr.reload_tuning(); the
    previous values are restored (and re-read) when the test ends."""

    def __init__(self):
        self._saved = {}

    def _reload(self):
        import collective_communication_reduction_way_amd as rr

        rr.reload_tuning()

    def set(self, name, value):
        self._saved.setdefault(name, os.environ.get(name))
        os.environ[name] = str(value)
        self._reload()

    def unset(self, name):
        self._saved.setdefault(name, os.environ.get(name))
        os.environ.pop(name, None)
        self._reload()

    def restore(self):
        if not self._saved:
            return
        for name, value in self._saved.items():
            if value is None:
                os.environ.pop(name, None)
            else:
                os.environ[name] = value
        self._saved.clear()
        self._reload()


@pytest.fixture
def tuning():
    t = TuningEnv()
    yield t
    t.restore()
