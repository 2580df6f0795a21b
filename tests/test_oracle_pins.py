"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
