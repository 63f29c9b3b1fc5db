"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each pin is a plain function taking the oracle's ctypes library and raising
AssertionError when the oracle disagrees with a closed form, an identity that
reduces to a textbook operation, or an invariant of the definition.  The same
functions run against copies of the oracle built with a planted mistake (see
test_oracle_mutants.py), to show that each plausible mistake fails at least one
of them.

Definition being pinned (Ascend HSTU blog, §1 formula; §3.2 causal diagonal; §4.2 jagged layout):
    out[r] = (1/n) * sum_{c <= r, same sequence} silu(alpha <q_r, k_c>) v_c
"""
from __future__ import annotations

import math
import os
from typing import Dict, List

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.txt")


# ---------------------------------------------------------------------------
# Golden hand-worked cases
# ---------------------------------------------------------------------------

def _sig(x: float) -> float:
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def _eval(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"exp": math.exp, "sig": _sig}))


def _parse_tokens(text: str, heads: int, d: int, evaluate) -> np.ndarray:
    toks = [t.strip() for t in text.split(";")]
    rows = []
    for t in toks:
        hs = [h.strip() for h in t.split("|")]
        if len(hs) != heads:
            raise ValueError(f"expected {heads} heads in {t!r}")
        row = []
        for h in hs:
            vals = h.split()
            if len(vals) != d:
                raise ValueError(f"expected {d} values in {h!r}")
            row.append([evaluate(x) for x in vals])
        rows.append(row)
    return np.array(rows, dtype=np.float64)


def golden_cases(path: str = GOLDEN) -> List[Dict]:
    cases, cur = [], None
    with open(path, encoding="utf-8") as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest.strip()}
            elif key == "end":
                cases.append(cur)
                cur = None
            else:
                cur[key] = rest.strip()
    out = []
    for c in cases:
        heads, d = int(c["heads"]), int(c["d"])
        offsets = np.array([int(x) for x in c["offsets"].split()], dtype=np.int32)
        T = int(offsets[-1])
        arrs = {}
        for name in ("q", "k", "v"):
            arrs[name] = (_parse_tokens(c[name], heads, d, float) if T else
                          np.zeros((0, heads, d)))
        expect = _parse_tokens(c["expect"], heads, d, _eval) if T else np.zeros((0, heads, d))
        targets = (np.array([int(x) for x in c["targets"].split()], dtype=np.int32)
                   if "targets" in c else None)
        out.append(dict(name=c["name"], heads=heads, d=d, offsets=offsets, targets=targets,
                        alpha=float(c["alpha"]), n=float(c["n"]), expect=expect, **arrs))
    return out


def pin_hand_worked(lib) -> None:
    """Closed-form hand-worked cases, in every storage type (all inputs are
    small dyadic numbers, exact in bf16, fp16 and fp32)."""
    for c in golden_cases():
        for dtype in ("fp32", "fp16", "bf16"):
            q, k, v = (workloads.cast_values(c[x].astype(np.float32), dtype)
                       for x in ("q", "k", "v"))
            got = oracle.fwd(q, k, v, c["offsets"], c["heads"], c["d"], c["alpha"], c["n"],
                             dtype, lib=lib)
            err = np.max(np.abs(got - c["expect"])) if got.size else 0.0
            scale = max(1.0, float(np.max(np.abs(c["expect"])))) if got.size else 1.0
            assert err <= 1e-13 * scale, (c["name"], dtype, err, got, c["expect"])


# ---------------------------------------------------------------------------
# SiLU shape: one-token sequences read the nonlinearity off directly
# ---------------------------------------------------------------------------

SILU_POINTS = [0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0, 7.25, -7.25, 10.0, -10.0,
               30.0, -30.0, 88.0, -88.0, 100.0, -100.0, 700.0, -700.0, 2.0 ** -20,
               -(2.0 ** -20)]


def _silu_textbook(x: float) -> float:
    return x * _sig(x)


def pin_silu_points(lib) -> None:
    """With one token per sequence, q = 1, v = 1, alpha = 1, n = 1, the output
    of sequence i is silu(k_i) exactly.  Compare with x / (1 + e^-x)."""
    pts = np.array(SILU_POINTS, dtype=np.float32)
    m = len(pts)
    offsets = np.arange(m + 1, dtype=np.int32)
    q = np.ones((m, 1, 1), np.float32)
    v = np.ones((m, 1, 1), np.float32)
    k = pts.reshape(m, 1, 1)
    got = oracle.fwd(q, k, v, offsets, 1, 1, 1.0, 1.0, "fp32", lib=lib).reshape(-1)
    for x, g in zip(pts, got):
        want = _silu_textbook(float(x))
        assert abs(g - want) <= 1e-14 * max(1.0, abs(want)), (float(x), g, want)


# ---------------------------------------------------------------------------
# Identities that reduce to textbook operations
# ---------------------------------------------------------------------------

def _rand_case(seed: int, lengths, heads: int, d: int, alpha: float, n: float):
    return workloads.make_case(lengths, heads, d, "fp32", seed, alpha=alpha, n=n)


def pin_sign_flip(lib) -> None:
    """silu(x) - silu(-x) = x, so hstu(Q) - hstu(-Q) = (alpha/n) tril(Q K^T) V,
    a masked matrix product computed here with numpy's matmul and tril."""
    c = _rand_case(11, [1, 5, 17, 0, 33, 2], 3, 8, 0.3, 7.0)
    a = oracle.fwd(c.q, c.k, c.v, c.offsets, c.heads, c.d, c.alpha, c.n, "fp32", lib=lib)
    b = oracle.fwd(-c.q, c.k, c.v, c.offsets, c.heads, c.d, c.alpha, c.n, "fp32", lib=lib)
    lhs = a - b
    Q, K, V = (x.astype(np.float64) for x in (c.q, c.k, c.v))
    rhs = np.zeros_like(lhs)
    off = c.offsets
    for i in range(c.num_seqs):
        s0, s1 = int(off[i]), int(off[i + 1])
        for h in range(c.heads):
            S = Q[s0:s1, h, :] @ K[s0:s1, h, :].T
            rhs[s0:s1, h, :] = (c.alpha / c.n) * (np.tril(S) @ V[s0:s1, h, :])
    err = np.max(np.abs(lhs - rhs))
    assert err <= 1e-12 * max(1.0, np.max(np.abs(rhs))), err


def pin_constant_rows(lib) -> None:
    """All q rows equal q*, all k rows equal k*: every score is the same, so
    out[r] = silu(alpha <q*,k*>)/n * (prefix sum of V up to r)."""
    rng = np.random.default_rng(5)
    lengths, heads, d, alpha, n = [4, 1, 9, 0, 6], 2, 5, 0.7, 3.0
    off = workloads.offsets_from_lengths(lengths)
    T = int(off[-1])
    qs = rng.standard_normal((heads, d)).astype(np.float32)
    ks = rng.standard_normal((heads, d)).astype(np.float32)
    q = np.broadcast_to(qs, (T, heads, d)).copy()
    k = np.broadcast_to(ks, (T, heads, d)).copy()
    v = rng.standard_normal((T, heads, d)).astype(np.float32)
    got = oracle.fwd(q, k, v, off, heads, d, alpha, n, "fp32", lib=lib)
    want = np.zeros_like(got)
    for h in range(heads):
        x = alpha * float(np.dot(qs[h].astype(np.float64), ks[h].astype(np.float64)))
        w = _silu_textbook(x) / n
        for i in range(len(lengths)):
            s0, s1 = int(off[i]), int(off[i + 1])
            want[s0:s1, h, :] = w * np.cumsum(v[s0:s1, h, :].astype(np.float64), axis=0)
    err = np.max(np.abs(got - want))
    assert err <= 1e-12 * max(1.0, np.max(np.abs(want))), err


def pin_first_rows(lib) -> None:
    """Row 0 of every sequence sees only itself: silu(alpha <q0,k0>) v0 / n."""
    c = _rand_case(21, [3, 1, 8, 2], 2, 4, 0.45, 5.0)
    got = oracle.fwd(c.q, c.k, c.v, c.offsets, c.heads, c.d, c.alpha, c.n, "fp32", lib=lib)
    for i in range(c.num_seqs):
        t = int(c.offsets[i])
        for h in range(c.heads):
            x = c.alpha * float(np.dot(c.q[t, h].astype(np.float64), c.k[t, h].astype(np.float64)))
            want = _silu_textbook(x) * c.v[t, h].astype(np.float64) / c.n
            assert np.max(np.abs(got[t, h] - want)) <= 1e-13 * max(1.0, np.max(np.abs(want)))


# ---------------------------------------------------------------------------
# Invariants of the definition
# ---------------------------------------------------------------------------

def pin_invariants(lib) -> None:
    c = _rand_case(31, [6, 0, 11, 3], 2, 6, 0.5, 4.0)

    def run(q, k, v, n=c.n, offsets=None):
        return oracle.fwd(q, k, v, c.offsets if offsets is None else offsets, c.heads, c.d,
                          c.alpha, n, "fp32", lib=lib)

    base = run(c.q, c.k, c.v)
    # K = 0: every score is 0 and silu(0) = 0.
    assert np.all(run(c.q, np.zeros_like(c.k), c.v) == 0.0)
    # Linear in V (dyadic values with few bits, so the fp32 sums are exact).
    v1 = np.round(c.v * 8.0) / 8.0
    v2 = np.round(workloads.make_case([int(x) for x in c.lengths], c.heads, c.d, "fp32",
                                      32).v * 8.0) / 8.0
    lin = run(c.q, c.k, v1 + v2) - (run(c.q, c.k, v1) + run(c.q, c.k, v2))
    assert np.max(np.abs(lin)) <= 1e-12 * max(1.0, np.max(np.abs(base))), np.max(np.abs(lin))
    # Halving n doubles the output exactly (power-of-two scaling).
    assert np.array_equal(run(c.q, c.k, c.v, n=c.n / 2), 2.0 * base)
    # Causality: changing k and v at local position p of sequence 2 only moves
    # rows >= p of that sequence.
    s0, p = int(c.offsets[2]), 4
    k3, v3 = c.k.copy(), c.v.copy()
    k3[s0 + p] += 1.0
    v3[s0 + p] -= 2.0
    moved = np.any(run(c.q, k3, v3) != base, axis=(1, 2))
    expect = np.zeros(c.total, bool)
    expect[s0 + p:int(c.offsets[3])] = True
    assert np.array_equal(moved, expect), (moved, expect)
    # Sequences are independent: one call per sequence gives the same bits,
    # and reordering sequences reorders the output segments.
    for i in range(c.num_seqs):
        a, b = int(c.offsets[i]), int(c.offsets[i + 1])
        one = oracle.fwd(c.q[a:b], c.k[a:b], c.v[a:b], np.array([0, b - a], np.int32),
                         c.heads, c.d, c.alpha, c.n, "fp32", lib=lib)
        assert np.array_equal(one, base[a:b])
    order = [2, 0, 3, 1]
    segs = [(int(c.offsets[i]), int(c.offsets[i + 1])) for i in order]
    perm = np.concatenate([np.arange(a, b) for a, b in segs]).astype(np.int64)
    off2 = workloads.offsets_from_lengths([b - a for a, b in segs])
    got = run(c.q[perm], c.k[perm], c.v[perm], offsets=off2)
    assert np.array_equal(got, base[perm])


# ---------------------------------------------------------------------------
# Brute force: the dense pair-set evaluation on tiny inputs
# ---------------------------------------------------------------------------

def pin_dense_bruteforce(lib) -> None:
    """The loop oracle against the dense evaluation over every (row, key)
    pair (einsum scores, boolean visibility matrix), on tiny inputs in every
    dtype."""
    specs = [([1], 1, 1), ([2, 3], 1, 2), ([16, 1, 0, 7, 5], 3, 8), ([9, 4], 2, 3)]
    for dtype in ("fp32", "fp16", "bf16"):
        for seed, (lengths, heads, d) in enumerate(specs):
            c = workloads.make_case(lengths, heads, d, dtype, 100 + seed, alpha=0.37, n=6.0)
            a = oracle.fwd(c.q, c.k, c.v, c.offsets, heads, d, c.alpha, c.n, dtype, lib=lib)
            b = oracle.dense_pairs(c.q, c.k, c.v, c.offsets, heads, d, c.alpha, c.n, dtype)
            err = np.max(np.abs(a - b))
            assert err <= 1e-12 * max(1.0, np.max(np.abs(b))), (dtype, lengths, err)


def pin_sampled_rows_match(lib) -> None:
    """The sampled-row entry point returns the same values as the full one."""
    c = workloads.make_case([5, 0, 12, 1, 30], 3, 16, "bf16", 41, alpha=0.25, n=30.0)
    full = oracle.fwd(c.q, c.k, c.v, c.offsets, c.heads, c.d, c.alpha, c.n, "bf16", lib=lib)
    rng = np.random.default_rng(0)
    tok = rng.integers(0, c.total, size=40)
    hd = rng.integers(0, c.heads, size=40)
    got = oracle.rows(c.q, c.k, c.v, c.offsets, c.heads, c.d, c.alpha, c.n, "bf16", tok, hd,
                      lib=lib)
    assert np.array_equal(got, full[tok, hd])


ALL_PINS = [pin_hand_worked, pin_silu_points, pin_sign_flip, pin_constant_rows,
            pin_first_rows, pin_invariants, pin_dense_bruteforce, pin_sampled_rows_match]
