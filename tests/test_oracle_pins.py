"""Pins of the CPU oracle against hand-worked values, exact rationals, closed forms and library conversions."""
import pytest

from oracle import lsa_oracle as O
from tests import oracle_checks as C


@pytest.mark.parametrize("check", C.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(O)
