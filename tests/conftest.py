import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; parity against the oracle")
    config.addinivalue_line(
        "markers", "slow: takes more than a few seconds (CPU pins, the GPU parity sweep)")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle._load()          # builds liboracle.so only when it is missing
    return oracle
