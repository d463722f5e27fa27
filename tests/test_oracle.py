"""The CPU oracle against the pages' printed values, closed forms, torch's fp64
SDPA and softmax-attention invariants (no GPU)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())
