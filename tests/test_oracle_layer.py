"""The oracle's layer surroundings against their pins, and three planted
mistakes (ORACLE_PLANT=15: U and V swapped in the split; 16: unbiased
variance in the layer norm; 17: residual dropped), each caught by at least
one pin."""
import os

import pytest

import oracle
import pins_layer


@pytest.mark.parametrize("pin", pins_layer.LAYER_PINS, ids=lambda p: p.__name__)
def test_layer_pin(pin):
    pin(oracle.load())


PLANTS = {15: "U and V swapped", 16: "unbiased variance", 17: "residual dropped"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_layer_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in pins_layer.LAYER_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {PLANTS[plant]!r} passed every pin"
