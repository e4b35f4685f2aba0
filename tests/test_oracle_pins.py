"""The oracle against its pins (CPU only)."""
import pytest

import oracle.fmlp_oracle as fo
from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(fo)
