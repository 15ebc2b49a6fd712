"""The CPU oracle against the pages' printed values, closed forms, invariants,
special cases and brute force (see ``oracle_pins.py`` for the sources)."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
