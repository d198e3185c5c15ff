"""The oracle against what the pages and mathematics fix (CPU only)."""

import pytest

import oracle.sdpa_oracle as so
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(so)


from tests.oracle_pins import BACKWARD_PINS  # noqa: E402


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=[p.__name__ for p in BACKWARD_PINS])
def test_backward_pin(pin):
    import oracle.sdpa_backward as sb

    pin(sb)


from tests.oracle_pins import DROPOUT_PINS  # noqa: E402


@pytest.mark.parametrize("pin", DROPOUT_PINS, ids=[p.__name__ for p in DROPOUT_PINS])
def test_dropout_pin(pin):
    import oracle.sdpa_dropout as sd

    pin(sd)
