"""The fp64 oracle against references other than itself (CPU only)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(0)
