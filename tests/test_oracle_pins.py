"""The CPU oracle against its pins (no GPU)."""
import pytest

from oracle import hisparse_oracle as ora
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ora)
