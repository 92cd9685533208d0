"""The oracle against its pins (closed forms, brute force, library special cases)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("check", pins.ALL, ids=[c.__name__ for c in pins.ALL])
def test_pin(o, check):
    check(o)
