"""The oracle against the pages' printed values and closed forms (CPU only)."""
import pytest

import oracle
from pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
