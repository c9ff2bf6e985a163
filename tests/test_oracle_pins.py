"""Runs every pin of tests/oracle_pins.py against the CPU oracle."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
