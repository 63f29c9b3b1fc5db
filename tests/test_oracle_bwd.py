"""The oracle's backward against its pins, and four planted backward mistakes
(ORACLE_PLANT=11: the sigmoid taken for silu's derivative; 12: dk built from k
instead of q; 13: alpha dropped from the chain rule; 14: key gradients taking
keys above the diagonal), each caught by at least two pins."""
import os

import pytest

import oracle
import pins_bwd


@pytest.mark.parametrize("pin", pins_bwd.BWD_PINS, ids=lambda p: p.__name__)
def test_bwd_pin(pin):
    pin(oracle.load())


PLANTS = {11: "sigmoid for silu'", 12: "dk from k", 13: "alpha dropped", 14: "mask ignored in dk/dv"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_bwd_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in pins_bwd.BWD_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert len(caught) >= 2, f"planted mistake {PLANTS[plant]!r} caught only by {caught}"
