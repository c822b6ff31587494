"""The oracle against its pins (see ``oracle_pins``)."""
import pytest
import torch

import oracle
from oracle_pins import PINS

torch.set_default_dtype(torch.float64)


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name](oracle)
