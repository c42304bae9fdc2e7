import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and libibp.so")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def orc():
    """The C oracle (built from oracle/ibp_oracle.c if needed)."""
    from oracle import build, oracle
    if not os.path.exists(oracle.DEFAULT_LIB):
        build.build()
    return oracle.default()


@pytest.fixture(scope="session")
def bmi2(tmp_path_factory):
    """The BMI2 helper of tests/helpers/bmi2_helper.c, built with gcc -mbmi2."""
    from tests.helpers import bmi2
    return bmi2.load(str(tmp_path_factory.mktemp("bmi2")))
