"""The oracle's target-aware (M-FALCON) mask against its pins, and the two
planted target-mask mistakes (ORACLE_PLANT=7: candidates see each other;
8: a candidate misses itself) each caught by at least two of them."""
import os

import pytest

import oracle
import pins_targets


@pytest.mark.parametrize("pin", pins_targets.TARGET_PINS, ids=lambda p: p.__name__)
def test_target_pin(pin):
    pin(oracle.load())


PLANTS = {7: "candidates see each other", 8: "candidate misses itself"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_target_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in pins_targets.TARGET_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert len(caught) >= 2, f"planted mistake {PLANTS[plant]!r} caught only by {caught}"
