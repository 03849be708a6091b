"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle.hybrid_oracle as O
from tests.oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_pin(check):
    check(O)
