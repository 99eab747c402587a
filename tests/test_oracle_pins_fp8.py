"""The FP8 (E4M3) oracle against the format's definition, torch's float8
conversions, brute force, scaling invariants and the 16-bit oracle (CPU only)."""

import pytest

import oracle.kv_fp8 as fp8_mod
from oracle_pins_fp8 import FP8_PINS


@pytest.mark.parametrize("pin", FP8_PINS, ids=[p.__name__ for p in FP8_PINS])
def test_fp8_oracle_pin(pin):
    pin(fp8_mod)
