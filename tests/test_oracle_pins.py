"""The oracle agrees with every pin (closed forms, a library routine, invariants)."""
import pytest

from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check, oracle_lib):
    check(oracle_lib)
