"""The f64 oracle against its pins (page-printed values, closed forms,
invariants, library routines, exact arithmetic). CPU only."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, pin):
    pin(oracle)
