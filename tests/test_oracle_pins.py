"""The oracle against its pins (CPU only)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)
