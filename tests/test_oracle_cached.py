"""The oracle's cached-history form against its pins, and the two planted
mistakes of that form (ORACLE_PLANT=9: the last history key missed; 10: a
candidate misses itself) each caught by at least two of them."""
import os

import pytest

import oracle
import pins_cached


@pytest.mark.parametrize("pin", pins_cached.CACHED_PINS, ids=lambda p: p.__name__)
def test_cached_pin(pin):
    pin(oracle.load())


PLANTS = {9: "last history key missed", 10: "candidate misses itself"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_cached_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in pins_cached.CACHED_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert len(caught) >= 2, f"planted mistake {PLANTS[plant]!r} caught only by {caught}"
