"""The fp64 oracle against the pins in ``pins.py`` (CPU only)."""
import pytest

from tests import pins, pins_bwd, pins_decode


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


@pytest.mark.parametrize("pin", pins_bwd.BWD_PINS, ids=lambda f: f.__name__)
def test_oracle_backward_pin(pin, oracle_lib):
    pin(oracle_lib)


@pytest.mark.parametrize("pin", pins_decode.DECODE_PINS, ids=lambda f: f.__name__)
def test_oracle_decode_pin(pin, oracle_lib):
    pin(oracle_lib)
