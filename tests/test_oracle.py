"""The CPU oracle against its pins (no GPU)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()


@pytest.mark.parametrize("seed", [1, 2])
def test_brute_force_more_seeds(seed):
    from oracle_pins import pin_brute_force, pin_sdpa
    pin_brute_force(seed)
    pin_sdpa(seed)
