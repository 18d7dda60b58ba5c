"""Pins of the oracle's decode, addressing, RoPE and down-projection (CPU only)."""

import pytest

import oracle_pins as P
from oracle import mla_oracle as orc


@pytest.mark.parametrize("pin", P.ALL_DECODE_PINS + [P.pin_paged_rows, P.pin_rope]
                         + P.PROJECTION_PINS,
                         ids=lambda f: f.__name__)
def test_pin(pin):
    pin(orc)
