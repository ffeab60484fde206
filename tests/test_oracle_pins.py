"""The CPU oracle pinned against library decoders, published format points,
exhaustive rounding search, exact rational sums, integer-exact cases and
invariants (see tests/oracle_pins.py for what each pin compares against)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
