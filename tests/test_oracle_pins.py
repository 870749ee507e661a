"""The oracle against its pins (CPU only).  See oracle_pin_checks.py."""
import pytest

import oracle
from tests import oracle_pin_checks as pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_pin(lib, check):
    check(lib)
