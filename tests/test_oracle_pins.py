"""The CPU oracle against the pages' worked examples, closed forms and brute force."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
