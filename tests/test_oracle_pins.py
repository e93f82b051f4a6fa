"""The oracle pinned to brute force, library routines, closed forms and the
pages' invariants (CPU only)."""
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
