"""The CPU oracle against the pages' worked examples, closed forms, invariants and a
50-digit brute force (no GPU)."""
import pytest

import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(oracle, check):
    check(oracle)
