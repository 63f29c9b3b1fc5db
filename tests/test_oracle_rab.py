"""The oracle's relative-attention-bias form against its pins, and the five
planted mistakes of that form (ORACLE_PLANT=18: bias scaled by alpha; 19:
relative position off by one; 20: time bucket of log2(gap) instead of
log2(gap + 1); 21: bias added after SiLU; 24: candidates keep their own
positions under the target-aware mask) each caught by at least two pins."""
import os

import pytest

import oracle
import pins_rab


@pytest.mark.parametrize("pin", pins_rab.RAB_PINS, ids=lambda p: p.__name__)
def test_rab_pin(pin):
    pin(oracle.load())


PLANTS = {18: "bias scaled by alpha", 19: "relative position off by one",
          20: "time bucket of log2(gap)", 21: "bias added after SiLU",
          24: "candidates keep their own positions"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_rab_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in pins_rab.RAB_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert len(caught) >= 2, f"planted mistake {PLANTS[plant]!r} caught only by {caught}"
