"""The CPU oracle against its pins (closed forms, identities, invariants)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_golden_file_parses():
    names = [c["name"] for c in pins.golden_cases()]
    assert {"two_token", "three_token_jagged", "three_token_one_sequence", "two_heads",
            "empty_and_single"} <= set(names)


def test_oracle_rejects_bad_offsets(lib):
    import numpy as np
    q = np.zeros((4, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, np.array([0, 3, 2, 4], np.int32), 1, 2, 1.0, 1.0, "fp32", lib=lib)
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, np.array([1, 4], np.int32), 1, 2, 1.0, 1.0, "fp32", lib=lib)
