"""The CPU oracle against hand-worked cases, closed forms, brute force,
invariants, exact rational arithmetic and library special cases."""
import pytest

from tests import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS,
                         ids=[c.__name__ for c in pins.ALL_CHECKS])
def test_oracle_pin(orc, check):
    check(orc)
