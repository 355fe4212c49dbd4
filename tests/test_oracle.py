"""The fp64 oracle against its pins (CPU only).  See tests/oracle_pins.py for what each pin is."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    err, tol = pin(oracle_lib)
    assert err <= tol, f"{pin.__name__}: error {err:.3e} > tolerance {tol:.1e}"
