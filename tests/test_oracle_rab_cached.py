"""The oracle's cached-history form with the relative attention bias against
its pins, and two planted mistakes (ORACLE_PLANT=26: candidates spread over
positions instead of all sitting right after the history; 27: the time gap
taken the other way), each caught by at least two pins."""
import os

import pytest

import oracle
import pins_rab_cached


@pytest.mark.parametrize("pin", pins_rab_cached.RAB_CACHED_PINS, ids=lambda p: p.__name__)
def test_rab_cached_pin(pin):
    pin(oracle.load())


PLANTS = {26: "candidates spread over positions", 27: "time gap taken the other way"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_rab_cached_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in pins_rab_cached.RAB_CACHED_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert len(caught) >= 2, f"planted mistake {PLANTS[plant]!r} caught only by {caught}"
