"""The oracle against brute force, closed forms, library routines and
hand-worked fixtures (CPU only)."""

import pytest

from oracle import nsa_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(O)
