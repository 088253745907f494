"""The CPU oracle against closed forms, invariants, hand-worked fixtures and
an independent dense float64 formulation (see ``pins.py``)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)
