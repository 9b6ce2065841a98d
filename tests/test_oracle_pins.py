"""The CPU oracle against what the pages and the mathematics fix (see tests/pins.py)."""
import pytest

import oracle
from pins import ALL_PINS


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(o, pin):
    pin(o)


def test_oracle_rejects_bad_arguments(o):
    import ctypes
    rc = o.lib.ss_oracle_scan(1, 1, 0, 1, *([None] * 9), 0, None, None, 1)
    assert rc == -1
    rc = o.lib.ss_oracle_scan(1, 1, 4, 8, *([None] * 9), 0, None, None, 1)
    assert rc == -1
    rc = o.lib.ss_oracle_state_update(1, 1, 65, None, *([None] * 8), 0, None, 1)
    assert rc == -1
