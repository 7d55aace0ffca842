"""The CPU oracle against brute force, closed forms, invariants and textbook routines."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pinned(check):
    check(P.real_impl())
