"""Pins for the oracle's gradients of the relative-attention-bias forward
under the target-aware (M-FALCON) mask (HSTU paper translation, §3.4: the mask
and rab_{p,t} change together; Appendix H, Algorithm 1 and Fig. 11: the
candidates of a micro-batch give what separate passes over the history and
one candidate would give).

The gradients are the derivative of the pinned forward (`fwd_rab` with
`num_targets`).  Each pin raises AssertionError when the oracle disagrees with
central finite differences of that forward, with the causal gradients where
the mask reduces to the causal one (no candidate, or one: the last row then
sits right after its history anyway), or with the sum of the causal gradients
of separate passes, one over the history alone and one per candidate over the
history followed by that candidate.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def _rand_dout(lens, heads, d, dtype, seed):
    return workloads.make_case(lens, heads, d, dtype, seed=seed).q


def pin_rab_tgt_bwd_finite_differences(lib) -> None:
    """Central differences of sum(out * dout) against every gradient (fp32
    inputs, steps of 2^-10), with candidates at the end of two sequences and a
    position table shorter than some candidate distances."""
    lens, tg = [5, 3, 6, 1], [2, 0, 3, 1]
    case = workloads.make_case(lens, 2, 3, "fp32", seed=401, alpha=0.5, n=3.0)
    r = workloads.make_rab_inputs(case.offsets, 3, 4, seed=402, max_log_gap=6)
    dout = _rand_dout(lens, 2, 3, "fp32", 403)
    wpos, wtime = r.pos_bias.astype(np.float64), r.time_bias.astype(np.float64)
    tgt = np.array(tg, dtype=np.int32)

    def loss(q=None, k=None, v=None, wp=wpos, wt=wtime):
        out = oracle.fwd_rab(case.q if q is None else q, case.k if k is None else k,
                             case.v if v is None else v, case.offsets, r.timestamps, wp, wt,
                             2, 3, case.alpha, case.n, "fp32", lib=lib, num_targets=tgt)
        return float(np.sum(out * dout.astype(np.float64)))

    dq, dk, dv, dpos, dtime = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets,
                                             r.timestamps, wpos, wtime, 2, 3, case.alpha,
                                             case.n, "fp32", lib=lib, num_targets=tgt)
    h = 2.0 ** -10
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        base = getattr(case, name)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += np.float32(h)
            minus[idx] -= np.float32(h)
            step = float(plus[idx]) - float(minus[idx])
            fd = (loss(**{name: plus}) - loss(**{name: minus})) / step
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    for name, table, grad in (("pos", wpos, dpos), ("time", wtime, dtime)):
        for j in range(len(table)):
            plus, minus = table.copy(), table.copy()
            plus[j] += h
            minus[j] -= h
            if name == "pos":
                fd = (loss(wp=plus) - loss(wp=minus)) / (2 * h)
            else:
                fd = (loss(wt=plus) - loss(wt=minus)) / (2 * h)
            assert abs(fd - grad[j]) <= 1e-5 * max(1.0, abs(fd)), (name, j, fd, grad[j])


def pin_rab_tgt_bwd_zero_or_one_candidate_is_causal(lib) -> None:
    """With no candidate the mask is the causal one; with one, the candidate
    is the last row, whose distance to a history key c is already s - 1 - c:
    both give the causal gradients exactly."""
    lens = [7, 1, 0, 12]
    case = workloads.make_case(lens, 2, 64, "bf16", seed=411)
    r = workloads.make_rab_inputs(case.offsets, 9, 6, seed=412)
    dout = _rand_dout(lens, 2, 64, "bf16", 413)
    ref = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, 2, 64, case.alpha, case.n, "bf16", lib=lib)
    for t in (0, 1):
        got = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps,
                             r.pos_bias, r.time_bias, 2, 64, case.alpha, case.n, "bf16",
                             lib=lib, num_targets=np.full(len(lens), t, dtype=np.int32))
        for name, a, b in zip(("dq", "dk", "dv", "dpos", "dtime"), got, ref):
            assert np.array_equal(a, b), (t, name)


def pin_rab_tgt_bwd_separate_passes(lib) -> None:
    """Appendix H's equivalence carried to the gradients: the loss of the
    target-aware forward is the history rows' causal loss plus, per
    candidate, the last row's loss of a causal pass over the history followed
    by that candidate alone.  So every gradient (tables included) is the sum
    of those passes' causal gradients, each pass with dout kept on its own
    rows only."""
    heads, d, dtype = 2, 16, "fp32"
    lens, tg = [9, 6, 4], [3, 6, 0]
    case = workloads.make_case(lens, heads, d, dtype, seed=421, alpha=0.25, n=5.0)
    r = workloads.make_rab_inputs(case.offsets, 7, 5, seed=422, max_log_gap=8)
    dout = _rand_dout(lens, heads, d, dtype, 423)
    got = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, heads, d, case.alpha, case.n, dtype, lib=lib,
                         num_targets=np.array(tg, dtype=np.int32))
    want = [np.zeros_like(got[0]), np.zeros_like(got[1]), np.zeros_like(got[2]),
            np.zeros(len(r.pos_bias)), np.zeros(len(r.time_bias))]
    off = case.offsets
    for i, (s, t) in enumerate(zip(lens, tg)):
        s0, hist = int(off[i]), s - t
        # pass over the history alone (dout on every history row), then one
        # pass per candidate j over [history, j] (dout on the last row only)
        passes = [(list(range(s0, s0 + hist)), None)] if hist > 0 else []
        passes += [(list(range(s0, s0 + hist)) + [s0 + j], s0 + j) for j in range(hist, s)]
        for toks, cand in passes:
            toks = np.array(toks, dtype=np.int64)
            sub_dout = dout[toks].copy()
            if cand is not None:
                sub_dout[:-1] = 0
            sub = oracle.bwd_rab(case.q[toks], case.k[toks], case.v[toks], sub_dout,
                                 np.array([0, len(toks)], dtype=np.int32), r.timestamps[toks],
                                 r.pos_bias, r.time_bias, heads, d, case.alpha, case.n, dtype,
                                 lib=lib)
            for m in range(3):
                np.add.at(want[m], toks, sub[m])
            want[3] += sub[3]
            want[4] += sub[4]
    for name, a, b in zip(("dq", "dk", "dv", "dpos", "dtime"), got, want):
        scale = max(1.0, float(np.max(np.abs(b))))
        assert np.max(np.abs(a - b)) <= 1e-12 * scale, (name, float(np.max(np.abs(a - b))))


def pin_rab_tgt_bwd_rows_match(lib) -> None:
    """Sampled rows equal the full gradients' rows (history and candidate
    tokens, candidates at 32-row block edges)."""
    lens, tg = [40, 3, 70], [9, 3, 33]
    case = workloads.make_case(lens, 2, 64, "bf16", seed=431)
    r = workloads.make_rab_inputs(case.offsets, 50, 9, seed=432)
    dout = _rand_dout(lens, 2, 64, "bf16", 433)
    tgt = np.array(tg, dtype=np.int32)
    full = oracle.bwd_rab(case.q, case.k, case.v, dout, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 64, case.alpha, case.n, "bf16", lib=lib,
                          num_targets=tgt)
    toks = np.array([0, 30, 31, 39, 40, 42, 43, 79, 80, 112], dtype=np.int64)
    hds = np.array([1, 0, 1, 0, 1, 1, 0, 0, 1, 0], dtype=np.int32)
    for kind, g in zip(("dq", "dk", "dv"), full[:3]):
        got = oracle.bwd_rab_rows(case.q, case.k, case.v, dout, case.offsets, r.timestamps,
                                  r.pos_bias, r.time_bias, 2, 64, case.alpha, case.n, "bf16",
                                  kind, toks, hds, lib=lib, num_targets=tgt)
        assert np.array_equal(got, g[toks, hds]), kind


RAB_TGT_BWD_PINS = [pin_rab_tgt_bwd_finite_differences,
                    pin_rab_tgt_bwd_zero_or_one_candidate_is_causal,
                    pin_rab_tgt_bwd_separate_passes, pin_rab_tgt_bwd_rows_match]
