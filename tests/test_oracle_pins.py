"""The float64 oracle against what the pages and the mathematics fix (CPU)."""

import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()
