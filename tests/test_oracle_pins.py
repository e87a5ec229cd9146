"""The oracle against its pins (closed forms, library codecs, exact brute force)."""

import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(orc, check):
    check(orc)


def test_threads_reported(orc):
    assert orc.num_threads() >= 1
