"""The CPU oracle against facts that do not come from it (no GPU needed).

Each check lives in oracle_pins.py so that test_oracle_mutants.py can run the
same checks against deliberately broken copies of the oracle.
"""
import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(lib, check):
    fails = check(lib)
    assert not fails, "\n".join(fails[:10])


def test_reading_cases_exist():
    wts, y, exp = pins._reading_cases()
    assert len(exp) >= 8
