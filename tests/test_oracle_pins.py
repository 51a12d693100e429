"""The fp64 oracle against closed forms, invariants, brute force and torch SDPA."""
import pytest

import oracle
from tests.oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
