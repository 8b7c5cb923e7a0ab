"""The CPU oracle pinned to hand-computed values, library routines and closed forms."""
import pytest

import oracle
import oracle_pin_suite as suite


@pytest.mark.parametrize("pin", suite.ALL, ids=[p.__name__ for p in suite.ALL])
def test_oracle_pin(pin):
    pin(oracle.default())
