"""The CPU oracle against its pins (closed forms, torch's SDPA, exact 50-digit
evaluation, the carry algebra, the recovery trial, special cases)."""

import pytest

import oracle.attention as orc
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(orc)
