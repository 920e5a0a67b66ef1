"""The CPU oracle against its pins (closed forms, limits, exact arithmetic,
finite differences, autograd, identities).  CPU only."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_golden_fixture_matches_exact_closed_form():
    pins.golden_closed_form_exact()
