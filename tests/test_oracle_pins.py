"""The fp64 oracle against its pins (CPU only)."""
import os

import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    if os.environ.get("FA_TEST_ORACLE_LIB"):   # another build of the oracle (the sanitizer run)
        return oracle.Oracle(oracle.load(os.environ["FA_TEST_ORACLE_LIB"]))
    return oracle.Oracle(oracle.load())   # builds when missing or older than its source


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
