"""The oracle's straight-through linear backward against its pins (CPU only)."""
import pytest

import oracle
from backward_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_backward_pin(name):
    assert PINS[name](oracle), name
