"""The oracle's complex-A scan against its pins (CPU)."""
import pytest

import oracle
from oracle_complex_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_complex_pin(name):
    fn, tol = PINS[name]
    err = fn(oracle.selective_scan_complex)
    assert err <= tol, f"{name}: {err:.3e}"
