"""Each planted mistake in the oracle must fail at least one pin.

The oracle source carries compile-time switches (ORACLE_PLANT=1..6) that each
plant one plausible mistake: the causal diagonal dropped, a sign error inside
SiLU, alpha applied after SiLU, a transposed score operand, attention across
the sequence boundary, and the 1/n normaliser dropped.  Mutant copies are
built into a temporary directory; the parity library is never one of them.
"""
import os

import pytest

import oracle
import pins

PLANTS = {1: "diagonal dropped", 2: "sign inside silu", 3: "alpha after silu",
          4: "transposed scores", 5: "cross-sequence leakage", 6: "normaliser dropped"}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p])
def test_planted_mistake_is_caught(tmp_path, plant):
    path = oracle.build(os.path.join(str(tmp_path), f"libmutant{plant}.so"), plant=plant)
    lib = oracle.load(path)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {PLANTS[plant]!r} passed every pin"
