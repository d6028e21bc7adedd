"""The fp64 oracle against its pins (CPU only). See oracle_pins.py for what each pin fixes."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[f.__name__ for f in P.ALL_PINS])
def test_pin(pin):
    import oracle
    pin(oracle.load())
