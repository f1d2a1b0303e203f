"""The oracle against its pins (CPU only)."""
import pytest

from oracle.oracle import get
from tests import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(get())


def test_input_generator_nested():
    """The M sweep is nested: the first rows of a larger draw equal a smaller draw."""
    import numpy as np
    from synth_inputs import activations
    big = activations(64, 2560)
    small = activations(16, 2560)
    assert np.array_equal(big[:16].view(np.uint16), small.view(np.uint16))
