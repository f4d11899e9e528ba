"""The fp64 oracle against independent references (CPU only).

See tests/pins.py for what each pin fixes and why it is independent of the
oracle's own code."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def ora():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(ora, pin):
    pin(ora)
