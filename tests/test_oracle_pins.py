"""The CPU oracle against facts other than itself (see ``oracle_pins.py``)."""

import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
