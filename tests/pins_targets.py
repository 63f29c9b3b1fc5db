"""Pins for the oracle's target-aware (M-FALCON) mask.

Mask (HSTU paper translation, §3.4 and Appendix H, Algorithm 1 and Fig. 11):
the last t tokens of a sequence are candidates; the causal mask is kept and
candidates do not see each other, so row r sees key c iff c <= r and
(c < h or c == r), h = s - t.  Each pin raises AssertionError when the oracle
disagrees with a closed form, with the equivalence the appendix states, or
with an explicit mask built the way the algorithm builds it.
"""
from __future__ import annotations

import os

import numpy as np

import oracle
import workloads
from pins import golden_cases

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "falcon_hand_worked.txt")


def pin_targets_hand_worked(lib) -> None:
    """Closed-form cases, every storage type (inputs are small integers)."""
    for c in golden_cases(GOLDEN):
        for dtype in ("fp32", "fp16", "bf16"):
            q, k, v = (workloads.cast_values(c[x].astype(np.float32), dtype)
                       for x in ("q", "k", "v"))
            got = oracle.fwd(q, k, v, c["offsets"], c["heads"], c["d"], c["alpha"], c["n"],
                             dtype, lib=lib, num_targets=c["targets"])
            err = float(np.max(np.abs(got - c["expect"])))
            assert err <= 1e-13 * max(1.0, float(np.max(np.abs(c["expect"])))), \
                (c["name"], dtype, got.ravel(), c["expect"].ravel())


def pin_targets_separate_passes(lib) -> None:
    """Appendix H: one pass over history + candidates with this mask gives each
    candidate the result of its own causal pass over history + that candidate
    (where it is the last token), and leaves the history rows as a causal pass
    over the history alone."""
    rng = np.random.default_rng(31)
    heads, d = 2, 64
    for h, t in ((5, 3), (0, 2), (7, 1), (3, 0)):
        s = h + t
        case = workloads.make_case([s], heads, d, "fp32", seed=int(rng.integers(1 << 30)))
        full = oracle.fwd(case.q, case.k, case.v, case.offsets, heads, d, case.alpha, case.n,
                          "fp32", lib=lib, num_targets=[t])
        if h:
            hist = oracle.fwd(case.q[:h], case.k[:h], case.v[:h], [0, h], heads, d, case.alpha,
                              case.n, "fp32", lib=lib)
            assert np.allclose(full[:h], hist, rtol=0, atol=1e-14), ("history rows", h, t)
        for i in range(t):
            idx = list(range(h)) + [h + i]
            one = oracle.fwd(case.q[idx], case.k[idx], case.v[idx], [0, h + 1], heads, d,
                             case.alpha, case.n, "fp32", lib=lib)
            assert np.allclose(full[h + i], one[h], rtol=0, atol=1e-14), ("candidate", h, t, i)


def pin_targets_dense_mask(lib) -> None:
    """Against the dense pair-set evaluation, whose visibility matrix follows
    Algorithm 1 (lower-triangular, candidate-candidate entries cleared)."""
    case = workloads.make_case([6, 1, 0, 9, 4], 3, 64, "bf16", seed=41)
    tg = np.array([2, 1, 0, 9, 1], dtype=np.int32)
    got = oracle.fwd(case.q, case.k, case.v, case.offsets, 3, 64, case.alpha, case.n, "bf16",
                     lib=lib, num_targets=tg)
    ref = oracle.dense_pairs(case.q, case.k, case.v, case.offsets, 3, 64, case.alpha, case.n,
                               "bf16", num_targets=tg)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))


def pin_targets_counts(lib) -> None:
    """No candidates is the plain causal mask; counts are clamped to [0, s];
    sampled rows match the full output."""
    case = workloads.make_case([5, 8, 3], 2, 64, "fp16", seed=43)
    args = (case.q, case.k, case.v, case.offsets, 2, 64, case.alpha, case.n, "fp16")
    plain = oracle.fwd(*args, lib=lib)
    zero = oracle.fwd(*args, lib=lib, num_targets=[0, 0, 0])
    assert np.array_equal(plain, zero)
    a = oracle.fwd(*args, lib=lib, num_targets=[9, -4, 3])
    b = oracle.fwd(*args, lib=lib, num_targets=[5, 0, 3])
    assert np.array_equal(a, b)
    toks = np.array([0, 4, 5, 9, 12, 15], dtype=np.int64)
    hds = np.array([0, 1, 1, 0, 1, 0], dtype=np.int32)
    r = oracle.rows(*args, toks, hds, lib=lib, num_targets=[5, 0, 3])
    assert np.array_equal(r, b[toks, hds])


TARGET_PINS = [pin_targets_hand_worked, pin_targets_separate_passes, pin_targets_dense_mask,
               pin_targets_counts]
