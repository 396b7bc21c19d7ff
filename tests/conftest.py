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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-size CPU work (oracle at full workload sizes)")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    return oracle.get()


class Forcing:
    """Forces the library's route variant / expand order for one test (through
    moe_testing_force) and restores the automatic choice afterwards."""

    def __init__(self):
        self.r, self.o, self.w, self.used = "auto", "auto", 0, False

    def _apply(self):
        from moe_glue_amd import _binding

        self.used = True
        _binding.testing_force(self.r, self.o, self.w)

    def route(self, name: str):
        self.r = name
        self._apply()

    def order(self, name: str):
        self.o = name
        self._apply()

    def workgroups_per_group(self, n: int):
        self.w = n
        self._apply()


@pytest.fixture
def force():
    f = Forcing()
    yield f
    if f.used:
        f.r, f.o, f.w = "auto", "auto", 0
        f._apply()
