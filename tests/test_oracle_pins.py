"""The CPU oracle against its pins (closed forms, invariants, hand fixtures,
independent implementations).  See tests/pins.py for what each pin checks."""
import pytest

from oracle import tileq_ref
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(tileq_ref)
