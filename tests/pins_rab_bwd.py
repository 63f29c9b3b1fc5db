"""Pins for the oracle's gradients of the forward with the relative attention
bias (HSTU paper translation, Appendix G: the backward recomputes the
attention and the bias and accumulates the bias gradients).

The gradients are the derivative of the pinned forward (`fwd_rab`).  Each pin
raises AssertionError when the oracle disagrees with central finite
differences of that forward (every input, both tables), with a closed form
for one-token sequences, with the plain backward when the tables are zero, or
with the identity that both tables' gradients add up to the same total (each
kept pair's score gradient is credited once to a distance and once to a time
bucket).
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def _loss(case, r, wpos, wtime, dout, q=None, k=None, v=None, lib=None):
    out = oracle.fwd_rab(case.q if q is None else q, case.k if k is None else k,
                         case.v if v is None else v, case.offsets, r.timestamps, wpos, wtime,
                         case.heads, case.d, case.alpha, case.n, "fp32", lib=lib)
    return float(np.sum(out * dout.astype(np.float64)))


def pin_rab_bwd_finite_differences(lib) -> None:
    """Central differences of sum(out * dout) (fp32 inputs, steps of 2^-10,
    exact in fp32 at these magnitudes) against every gradient."""
    case = workloads.make_case([3, 1, 4], 2, 3, "fp32", seed=201, alpha=0.5, n=3.0)
    r = workloads.make_rab_inputs(case.offsets, 3, 4, seed=202, max_log_gap=6)
    dout = workloads.make_case([3, 1, 4], 2, 3, "fp32", seed=203).q
    wpos, wtime = r.pos_bias.astype(np.float64), r.time_bias.astype(np.float64)
    dq, dk, dv, dpos, dtime = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets,
                                             r.timestamps, wpos, wtime, 2, 3, case.alpha, case.n,
                                             "fp32", lib=lib)
    h = 2.0 ** -10
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        base = getattr(case, name)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += np.float32(h)
            minus[idx] -= np.float32(h)
            step = float(plus[idx]) - float(minus[idx])
            fd = (_loss(case, r, wpos, wtime, dout, lib=lib, **{name: plus}) -
                  _loss(case, r, wpos, wtime, dout, lib=lib, **{name: minus})) / step
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    for name, table, grad in (("pos", wpos, dpos), ("time", wtime, dtime)):
        for j in range(len(table)):
            plus, minus = table.copy(), table.copy()
            plus[j] += h
            minus[j] -= h
            args = (plus, wtime) if name == "pos" else (wpos, plus)
            argm = (minus, wtime) if name == "pos" else (wpos, minus)
            fd = (_loss(case, r, *args, dout, lib=lib) - _loss(case, r, *argm, dout, lib=lib)) / (2 * h)
            assert abs(fd - grad[j]) <= 1e-5 * max(1.0, abs(fd)), (name, j, fd, grad[j])


def pin_rab_bwd_single_token_closed_form(lib) -> None:
    """One-token sequences: out = silu(x) v / n, x = alpha <q, k> + wpos[0] +
    wtime[0], so d/dwpos[0] = d/dwtime[0] = sum over tokens and heads of
    silu'(x) <dout, v> / n, with silu'(x) = (1 + e^-x + x e^-x) / (1 + e^-x)^2."""
    case = workloads.make_case([1] * 5, 3, 8, "fp32", seed=211, n=2.0)
    r = workloads.make_rab_inputs(case.offsets, 2, 3, seed=212)
    dout = workloads.make_case([1] * 5, 3, 8, "fp32", seed=213).q
    _, _, _, dpos, dtime = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets,
                                          r.timestamps, r.pos_bias, r.time_bias, 3, 8,
                                          case.alpha, case.n, "fp32", lib=lib)
    q, k, v, do = (a.astype(np.float64) for a in (case.q, case.k, case.v, dout))
    x = case.alpha * np.sum(q * k, axis=-1) + float(r.pos_bias[0]) + float(r.time_bias[0])
    e = np.exp(-x)
    ds = (1.0 + e + x * e) / (1.0 + e) ** 2
    want = float(np.sum(ds * np.sum(do * v, axis=-1) / case.n))
    assert abs(dpos[0] - want) <= 1e-12 * max(1.0, abs(want)), (dpos, want)
    assert abs(dtime[0] - want) <= 1e-12 * max(1.0, abs(want)), (dtime, want)
    assert np.all(dpos[1:] == 0) and np.all(dtime[1:] == 0)


def pin_rab_bwd_zero_tables_is_plain(lib) -> None:
    """Zero tables: dq, dk, dv are the plain backward's."""
    case = workloads.make_case([6, 0, 19, 2], 2, 64, "bf16", seed=221)
    r = workloads.make_rab_inputs(case.offsets, 5, 7, seed=222)
    dout = workloads.make_case([6, 0, 19, 2], 2, 64, "bf16", seed=223).q
    got = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, np.zeros(5),
                         np.zeros(7), 2, 64, case.alpha, case.n, "bf16", lib=lib)
    ref = oracle.bwd(case.q, case.k, case.v, dout, case.offsets, 2, 64, case.alpha, case.n,
                     "bf16", lib=lib)
    for a, b in zip(got[:3], ref):
        assert np.max(np.abs(a - b)) <= 1e-13 * max(1.0, float(np.max(np.abs(b))))


def pin_rab_bwd_table_totals_agree(lib) -> None:
    """With a position entry for every distance (npos = the longest length),
    the two tables' gradients have the same total."""
    lens = [9, 14, 1, 5]
    case = workloads.make_case(lens, 2, 64, "fp16", seed=231, sigma=0.5)
    r = workloads.make_rab_inputs(case.offsets, 14, 6, seed=232)
    dout = workloads.make_case(lens, 2, 64, "fp16", seed=233, sigma=0.5).q
    _, _, _, dpos, dtime = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets,
                                          r.timestamps, r.pos_bias, r.time_bias, 2, 64,
                                          case.alpha, case.n, "fp16", lib=lib)
    assert abs(np.sum(dpos) - np.sum(dtime)) <= 1e-12 * max(1.0, float(np.sum(np.abs(dpos))))


def pin_rab_bwd_rows_match(lib) -> None:
    """Sampled rows equal the full gradients' rows."""
    case = workloads.make_case([30, 2, 45], 2, 128, "bf16", seed=241)
    r = workloads.make_rab_inputs(case.offsets, 20, 9, seed=242)
    dout = workloads.make_case([30, 2, 45], 2, 128, "bf16", seed=243).q
    full = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 128, case.alpha, case.n, "bf16", lib=lib)
    toks = np.array([0, 29, 30, 31, 32, 50, 76], dtype=np.int64)
    hds = np.array([1, 0, 1, 0, 1, 1, 0], dtype=np.int32)
    for kind, g in zip(("dq", "dk", "dv"), full[:3]):
        got = oracle.bwd_rab_rows(case.q, case.k, case.v, dout, case.offsets, r.timestamps,
                                  r.pos_bias, r.time_bias, 2, 128, case.alpha, case.n, "bf16",
                                  kind, toks, hds, lib=lib)
        assert np.array_equal(got, g[toks, hds]), kind


RAB_BWD_PINS = [pin_rab_bwd_finite_differences, pin_rab_bwd_single_token_closed_form,
                pin_rab_bwd_zero_tables_is_plain, pin_rab_bwd_table_totals_agree,
                pin_rab_bwd_rows_match]
