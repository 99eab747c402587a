"""The oracle against values the pages print, closed forms, torch's float64
attention, brute force and invariants (CPU only)."""

import pytest

import oracle.paged_attention as oracle_mod
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle_mod)
