"""The CPU oracle agrees with every pin (hand-worked example, closed forms, invariants,
library special cases, brute force). No GPU needed."""

import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
