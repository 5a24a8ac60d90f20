"""The fp64 oracle against its pins (CPU only)."""
import pytest

from oracle import gsi_oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(gsi_oracle)
