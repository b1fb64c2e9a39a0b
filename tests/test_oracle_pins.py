"""The CPU oracle against its pins (no GPU needed)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle
from oracle_pins import ALL_CHECKS


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_pin(check):
    check()
