"""The oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("name", sorted(pins.ALL_PINS))
def test_pin(name):
    pins.ALL_PINS[name]()
