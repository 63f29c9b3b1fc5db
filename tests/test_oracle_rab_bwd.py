"""The oracle's gradients of the relative-attention-bias forward (causal and
target-aware) against their pins, and planted mistakes (ORACLE_PLANT=22: the
bias gradient scaled by alpha; 23: the position gradient credited one
distance off; 24: candidates keep their own positions in the bias; 25:
candidates' position gradients credited at their own distances), each caught
by at least two pins."""
import os

import pytest

import oracle
import pins_rab_bwd
import pins_rab_bwd_targets

ALL_PINS = pins_rab_bwd.RAB_BWD_PINS + pins_rab_bwd_targets.RAB_TGT_BWD_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_rab_bwd_pin(pin):
    pin(oracle.load())


PLANTS = {22: "bias gradient scaled by alpha", 23: "position gradient one distance off",
          24: "candidates keep their own positions",
          25: "candidates' position gradient at their own distance"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_rab_bwd_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert len(caught) >= 2, f"planted mistake {PLANTS[plant]!r} caught only by {caught}"
