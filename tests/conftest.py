import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--random-shape-seeds", type=int, default=32,
                     help="how many seeded random shapes the randomized GPU parity test "
                          "draws (default 32)")
    parser.addoption("--random-shape-first", type=int, default=0,
                     help="the first seed of those shapes (default 0)")


def pytest_generate_tests(metafunc):
    if "random_seed" in metafunc.fixturenames:
        n = metafunc.config.getoption("--random-shape-seeds")
        first = metafunc.config.getoption("--random-shape-first")
        metafunc.parametrize("random_seed", range(first, first + n))


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity through the C ABI")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle
