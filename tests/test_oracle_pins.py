"""The CPU oracle against hand-worked cases, exact rational arithmetic,
closed forms, brute force and invariants (see pins.py)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)
