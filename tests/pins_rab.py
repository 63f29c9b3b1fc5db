"""Pins for the oracle's causal forward with the relative attention bias.

Source: HSTU paper translation, §3 (rab_{p,t} is added to the scores before
phi_2 = SiLU; it merges position and time) and Appendix G (the bias is built
inside the operator from its parameters).  The page's equation is lost; the
reading pinned here is
  rab(r, c) = wpos[r - c] + wtime[min(floor(log2(ts_r - ts_c + 1)), ntime - 1)]
(wpos[j] = 0 for j >= npos; a negative gap in the last bucket), added after
alpha.  Each pin raises AssertionError when the oracle disagrees with a
hand-worked case, with the plain forward on inputs that carry the bias as
extra head dimensions (a constant bias is one more dimension with q = 1; a
bias linear in r - c is two more), with a bucket found by floating-point
log2, or with an invariance the reading implies.
"""
from __future__ import annotations

import os

import numpy as np

import oracle
import workloads
from pins import _eval, _parse_tokens

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "rab_hand_worked.txt")


def rab_golden_cases(path: str = GOLDEN):
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
        ints = lambda key: np.array([int(x) for x in c[key].split()], dtype=np.int64)
        floats = lambda key: np.array([float(x) for x in c[key].split()], dtype=np.float64)
        out.append(dict(name=c["name"], heads=heads, d=d, offsets=ints("offsets").astype(np.int32),
                        ts=ints("ts").astype(np.int32), wpos=floats("wpos"),
                        wtime=floats("wtime"), alpha=float(c["alpha"]), n=float(c["n"]),
                        expect=_parse_tokens(c["expect"], heads, d, _eval),
                        **{x: _parse_tokens(c[x], heads, d, float) for x in ("q", "k", "v")}))
    return out


def _close(got, ref, tol=1e-13):
    return float(np.max(np.abs(got - ref))) <= tol * max(1.0, float(np.max(np.abs(ref))))


def pin_rab_hand_worked(lib) -> None:
    """Hand-worked cases, every storage type (inputs are exact in all three)."""
    for c in rab_golden_cases():
        for dtype in ("fp32", "fp16", "bf16"):
            q, k, v = (workloads.cast_values(c[x].astype(np.float32), dtype) for x in "qkv")
            got = oracle.fwd_rab(q, k, v, c["offsets"], c["ts"], c["wpos"], c["wtime"],
                                 c["heads"], c["d"], c["alpha"], c["n"], dtype, lib=lib)
            assert _close(got, c["expect"]), (c["name"], dtype, got.ravel(), c["expect"].ravel())


def _extended(case, cols_q, cols_k):
    """fp32 q, k, v with extra head dimensions appended per token (v gets
    zeros there); cols_* map (local row, sequence index) to the extra values."""
    T, H, d = case.q.shape
    extra = len(cols_q(0, 0))
    q = np.zeros((T, H, d + extra), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[:, :, :d], k[:, :, :d], v[:, :, :d] = case.q, case.k, case.v
    for i in range(case.num_seqs):
        a, b = int(case.offsets[i]), int(case.offsets[i + 1])
        for r in range(b - a):
            q[a + r, :, d:] = cols_q(r, i)
            k[a + r, :, d:] = cols_k(r, i)
    return q, k, v


def pin_rab_constant_bias_is_one_more_dimension(lib) -> None:
    """A bias that is the same for every pair (constant tables, every distance
    inside the position table) equals one more head dimension with q = 1 and
    k = bias / alpha, under the plain forward: the bias sits inside SiLU,
    after alpha."""
    lens = [7, 1, 12]
    case = workloads.make_case(lens, 2, 64, "fp32", seed=101, alpha=0.125, n=12.0)
    ts = workloads.make_rab_inputs(case.offsets, 12, 5, seed=102).timestamps
    wpos, wtime = np.full(12, 0.375), np.full(5, 0.125)     # bias 0.5 = 4 * alpha
    got = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, ts, wpos, wtime, 2, 64, case.alpha,
                         case.n, "fp32", lib=lib)
    q, k, v = _extended(case, lambda r, i: [1.0], lambda r, i: [4.0])
    ref = oracle.fwd(q, k, v, case.offsets, 2, 65, case.alpha, case.n, "fp32", lib=lib)[:, :, :64]
    assert _close(got, ref, 1e-12)


def pin_rab_linear_position_is_two_more_dimensions(lib) -> None:
    """wpos[j] = beta * j (every distance inside the table), no time term:
    alpha <q, k> + beta (r - c) = alpha <[q, r, 1], [k, beta/alpha, -c beta/alpha]>,
    so the plain forward on the extended inputs gives the same output (pins
    the direction r - c of the relative position)."""
    lens = [9, 16, 3]
    case = workloads.make_case(lens, 2, 64, "fp32", seed=111, alpha=0.125, n=16.0)
    ts = workloads.make_rab_inputs(case.offsets, 16, 3, seed=112).timestamps
    beta = 1.0 / 64.0                                           # beta / alpha = 1/8
    wpos, wtime = beta * np.arange(16), np.zeros(3)
    got = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, ts, wpos, wtime, 2, 64, case.alpha,
                         case.n, "fp32", lib=lib)
    q, k, v = _extended(case, lambda r, i: [float(r), 1.0], lambda r, i: [0.125, -0.125 * r])
    ref = oracle.fwd(q, k, v, case.offsets, 2, 66, case.alpha, case.n, "fp32", lib=lib)[:, :, :64]
    assert _close(got, ref, 1e-12)


def pin_rab_time_buckets_by_float_log2(lib) -> None:
    """Time buckets read back through the output: q = 0 and v_c = e_c make
    out[r][c] = silu(wtime[bucket] + wpos[r - c]) / n with wpos = 0; wtime[b] =
    b + 1 is distinct per bucket.  The expected bucket comes from numpy's
    floating-point log2 (exact at these sizes), gaps straddling powers of two."""
    gaps = [0, 1, 2, 3, 4, 6, 7, 8, 14, 15, 16, 62, 63, 64, 1022, 1023, 1024, 4095, 70000]
    ts = np.concatenate([[0], np.cumsum(gaps)]).astype(np.int32)
    s = len(ts)
    ntime = 12
    q = np.zeros((s, 1, s), np.float32)
    k = np.ones_like(q)
    v = np.eye(s, dtype=np.float32).reshape(s, 1, s)
    wtime = np.arange(1, ntime + 1, dtype=np.float64)
    got = oracle.fwd_rab(q, k, v, [0, s], ts, np.zeros(1), wtime, 1, s, 0.5, 3.0, "fp32",
                         lib=lib)[:, 0, :]
    t = ts.astype(np.float64)
    gap = t[:, None] - t[None, :]
    bucket = np.minimum(np.floor(np.log2(np.maximum(gap, 0) + 1)), ntime - 1)
    x = bucket + 1.0
    ref = np.tril(x / (1.0 + np.exp(-x)) / 3.0)
    assert _close(got, ref), np.argwhere(np.abs(got - ref) > 1e-12)


def pin_rab_zero_tables_is_plain(lib) -> None:
    """Zero tables give the plain causal forward (any timestamps)."""
    case = workloads.make_case([5, 33, 1, 20], 3, 64, "bf16", seed=121)
    ts = workloads.make_rab_inputs(case.offsets, 8, 4, seed=122).timestamps
    got = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, ts, np.zeros(8), np.zeros(4), 3,
                         64, case.alpha, case.n, "bf16", lib=lib)
    ref = oracle.fwd(case.q, case.k, case.v, case.offsets, 3, 64, case.alpha, case.n, "bf16",
                     lib=lib)
    assert _close(got, ref, 1e-14)


def pin_rab_relative_only(lib) -> None:
    """The bias depends on differences only: shifting one sequence's
    timestamps by a constant, or appending zero entries to the position table
    past every distance, changes nothing."""
    case = workloads.make_case([17, 6], 2, 64, "fp16", seed=131, sigma=0.5)
    r = workloads.make_rab_inputs(case.offsets, 10, 6, seed=132)
    base = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 64, case.alpha, case.n, "fp16", lib=lib)
    ts2 = r.timestamps.copy()
    ts2[:17] += 12345
    wp2 = np.concatenate([r.pos_bias, np.zeros(20, np.float32)])
    other = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, ts2, wp2, r.time_bias, 2, 64,
                           case.alpha, case.n, "fp16", lib=lib)
    assert np.array_equal(base, other)


def pin_rab_rows_match(lib) -> None:
    """Sampled rows equal the full output's rows."""
    case = workloads.make_case([40, 3, 70], 2, 128, "bf16", seed=141)
    r = workloads.make_rab_inputs(case.offsets, 50, 9, seed=142)
    full = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 128, case.alpha, case.n, "bf16", lib=lib)
    toks = np.array([0, 39, 40, 42, 43, 100, 112], dtype=np.int64)
    hds = np.array([0, 1, 1, 0, 1, 0, 1], dtype=np.int32)
    got = oracle.rows_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 128, case.alpha, case.n, "bf16", toks, hds, lib=lib)
    assert np.array_equal(got, full[toks, hds])


RAB_PINS = [pin_rab_hand_worked, pin_rab_constant_bias_is_one_more_dimension,
            pin_rab_linear_position_is_two_more_dimensions, pin_rab_time_buckets_by_float_log2,
            pin_rab_zero_tables_is_plain, pin_rab_relative_only, pin_rab_rows_match]


# ---- the bias under the target-aware mask (M-FALCON) ----------------------
# HSTU paper translation §3.4: M-FALCON changes the mask and rab_{p,t} so that
# the candidates of a micro-batch all run the same operations.  Reading: a
# candidate takes the position right after the history (distance hist - c to
# a history key, 0 to itself); timestamps stay its own.

def _targets_case(seed):
    lens, tgts = [9, 12, 5, 1], [3, 0, 5, 1]
    case = workloads.make_case(lens, 2, 64, "fp32", seed=seed, n=12.0)
    r = workloads.make_rab_inputs(case.offsets, 10, 8, seed=seed + 1)
    return case, r, np.array(tgts, np.int32)


def pin_rab_targets_candidate_is_history_plus_itself(lib) -> None:
    """Algorithm 1's equivalence: each candidate's row equals the last row of
    the causal bias forward over the history followed by that candidate alone
    (placed at position hist)."""
    case, r, tg = _targets_case(301)
    got = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, 2, 64, case.alpha, case.n, "fp32", lib=lib, num_targets=tg)
    checked = 0
    for i in range(case.num_seqs):
        a, b = int(case.offsets[i]), int(case.offsets[i + 1])
        hist = (b - a) - int(tg[i])
        for row in range(a + hist, b):
            idx = list(range(a, a + hist)) + [row]
            one = oracle.fwd_rab(case.q[idx], case.k[idx], case.v[idx], [0, hist + 1],
                                 r.timestamps[idx], r.pos_bias, r.time_bias, 2, 64, case.alpha,
                                 case.n, "fp32", lib=lib)
            assert np.allclose(got[row], one[hist], rtol=0, atol=1e-14), (i, row)
            checked += 1
    assert checked == 9


def pin_rab_targets_candidate_order(lib) -> None:
    """Reordering a sequence's candidates (their q, k, v and timestamps)
    reorders their outputs and changes nothing else."""
    case, r, tg = _targets_case(311)
    base = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 64, case.alpha, case.n, "fp32", lib=lib,
                          num_targets=tg)
    perm = np.arange(case.total)
    a, b = int(case.offsets[2]), int(case.offsets[3])   # 5 tokens, all candidates
    perm[a:b] = perm[a:b][::-1]
    a, b = int(case.offsets[0]), int(case.offsets[1])   # 9 tokens, the last 3 candidates
    perm[b - 3:b] = perm[b - 3:b][[2, 0, 1]]
    got = oracle.fwd_rab(case.q[perm], case.k[perm], case.v[perm], case.offsets,
                         r.timestamps[perm], r.pos_bias, r.time_bias, 2, 64, case.alpha, case.n,
                         "fp32", lib=lib, num_targets=tg)
    assert np.allclose(got, base[perm], rtol=0, atol=1e-14)


def pin_rab_targets_without_candidates_is_causal(lib) -> None:
    """No candidates: the causal bias forward."""
    case, r, _ = _targets_case(321)
    got = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, 2, 64, case.alpha, case.n, "fp32", lib=lib,
                         num_targets=np.zeros(4, np.int32))
    ref = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                         r.time_bias, 2, 64, case.alpha, case.n, "fp32", lib=lib)
    assert np.array_equal(got, ref)


def pin_rab_targets_rows_match(lib) -> None:
    case, r, tg = _targets_case(331)
    full = oracle.fwd_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 64, case.alpha, case.n, "fp32", lib=lib,
                          num_targets=tg)
    toks = np.arange(case.total, dtype=np.int64)
    hds = (toks % 2).astype(np.int32)
    got = oracle.rows_rab(case.q, case.k, case.v, case.offsets, r.timestamps, r.pos_bias,
                          r.time_bias, 2, 64, case.alpha, case.n, "fp32", toks, hds, lib=lib,
                          num_targets=tg)
    assert np.array_equal(got, full[toks, hds])


RAB_PINS += [pin_rab_targets_candidate_is_history_plus_itself, pin_rab_targets_candidate_order,
             pin_rab_targets_without_candidates_is_causal, pin_rab_targets_rows_match]
