"""The oracle against its pins (CPU only)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(orc, check):
    check(orc)
