"""The float64 oracle against its pins (closed forms, brute force, textbook
algorithms, finite differences, invariants).  CPU only."""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.pc_oracle)
