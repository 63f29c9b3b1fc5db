"""Pins for the oracle's cached-history form with the relative attention bias
(HSTU paper translation, Appendix H: a micro-batch of candidates attends to
the cached K and V of its request's history plus itself; §3.4: M-FALCON
moves the bias with the mask).  The reading: a candidate sits right after its
history of h cached keys (distance h - c to cached key c, 0 to itself) and
keeps its own timestamp.

Each pin raises AssertionError when the oracle disagrees with: the candidate
rows of the target-aware bias forward over each request's history followed by
its candidates (the pinned reading of §3.4); the cached form without bias
when both tables are zero; a closed form for one cached key; sampled rows.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def _case(hist, cand, heads, d, dtype, seed, npos=40, ntime=8, max_log_gap=10):
    cc = workloads.make_cached_case(hist, cand, heads, d, dtype, seed=seed)
    r, hts = workloads.make_cached_rab_inputs(cc.hist_offsets, cc.cand.offsets, npos, ntime,
                                              seed=seed + 1, max_log_gap=max_log_gap)
    return cc, r, hts


def _cached(cc, r, hts, lib, wpos=None, wtime=None):
    c = cc.cand
    return oracle.fwd_rab_cached(c.q, c.k, c.v, c.offsets, cc.k_cache, cc.v_cache,
                                 cc.hist_offsets, r.timestamps, hts,
                                 r.pos_bias if wpos is None else wpos,
                                 r.time_bias if wtime is None else wtime, c.heads, c.d, c.alpha,
                                 c.n, c.dtype, lib=lib)


def pin_rab_cached_equals_target_aware(lib) -> None:
    """Candidate rows = the target-aware bias forward over [history; candidates]
    (history rows' q set to zero: they are not compared), per request."""
    for dtype, d in (("fp32", 16), ("bf16", 64)):
        hist, cand = [0, 5, 37, 1, 64], [3, 1, 9, 4, 0]
        cc, r, hts = _case(hist, cand, 2, d, dtype, seed=601)
        got = _cached(cc, r, hts, lib)
        c = cc.cand
        lengths = [h + t for h, t in zip(hist, cand)]
        joint = workloads.offsets_from_lengths(lengths)
        T = int(joint[-1])
        qj = np.zeros((T, 2, d), dtype=c.q.dtype)
        kj, vj = np.zeros_like(qj), np.zeros_like(qj)
        tsj = np.zeros(T, dtype=np.int32)
        rows = []
        for i, (h, t) in enumerate(zip(hist, cand)):
            j0, h0, c0 = int(joint[i]), int(cc.hist_offsets[i]), int(c.offsets[i])
            kj[j0:j0 + h], vj[j0:j0 + h] = cc.k_cache[h0:h0 + h], cc.v_cache[h0:h0 + h]
            tsj[j0:j0 + h] = hts[h0:h0 + h]
            qj[j0 + h:j0 + h + t] = c.q[c0:c0 + t]
            kj[j0 + h:j0 + h + t], vj[j0 + h:j0 + h + t] = c.k[c0:c0 + t], c.v[c0:c0 + t]
            tsj[j0 + h:j0 + h + t] = r.timestamps[c0:c0 + t]
            rows += list(range(j0 + h, j0 + h + t))
        ref = oracle.fwd_rab(qj, kj, vj, joint, tsj, r.pos_bias, r.time_bias, 2, d, c.alpha, c.n,
                             dtype, lib=lib, num_targets=np.array(cand, np.int32))[rows]
        scale = max(1.0, float(np.max(np.abs(ref))))
        assert np.max(np.abs(got - ref)) <= 1e-12 * scale, (dtype, float(np.max(np.abs(got - ref))))


def pin_rab_cached_zero_tables_is_cached(lib) -> None:
    """Zero tables: exactly the cached-history form without bias."""
    cc, r, hts = _case([0, 7, 130], [2, 5, 33], 3, 64, "bf16", seed=611)
    got = _cached(cc, r, hts, lib, wpos=np.zeros(40), wtime=np.zeros(8))
    c = cc.cand
    ref = oracle.fwd_cached(c.q, c.k, c.v, c.offsets, cc.k_cache, cc.v_cache, cc.hist_offsets,
                            c.heads, c.d, c.alpha, c.n, c.dtype, lib=lib)
    assert np.array_equal(got, ref)


def pin_rab_cached_one_cached_key_closed_form(lib) -> None:
    """One cached key, four candidates (d = 2, fp32): candidate j's row is
    (silu(alpha <q_j, kc> + wpos[1] + wtime[b_j]) vc + silu(alpha <q_j, k_j> +
    wpos[0] + wtime[0]) v_j) / n, b_j = min(floor(log2(ts_j - ts_c + 1)),
    ntime - 1) from numpy's floating-point log2 (exact at these gaps)."""
    d = 2
    cc = workloads.make_cached_case([1], [4], 1, d, "fp32", seed=621, alpha=0.75, n=3.0)
    c = cc.cand
    hts = np.array([1000], dtype=np.int32)
    ts = np.array([1000, 1003, 1040, 5000], dtype=np.int32)      # gaps 0, 3, 40, 4000
    wpos = np.array([0.5, -1.25, 2.0, 3.5, -0.75, 1.5], dtype=np.float64)
    wtime = np.array([0.25, -0.5, 0.75, 1.0, -1.5, 2.25, 0.125, -0.25], dtype=np.float64)
    r = workloads.RabInputs(timestamps=ts, pos_bias=wpos, time_bias=wtime)
    got = _cached(cc, r, hts, lib)
    q, k, v = (x.astype(np.float64)[:, 0, :] for x in (c.q, c.k, c.v))
    kc, vc = (x.astype(np.float64)[0, 0, :] for x in (cc.k_cache, cc.v_cache))
    silu = lambda x: x / (1.0 + np.exp(-x))
    for j in range(4):
        b = min(int(np.floor(np.log2(float(ts[j] - hts[0]) + 1.0))), len(wtime) - 1)
        xh = c.alpha * float(q[j] @ kc) + wpos[1] + wtime[b]
        xs = c.alpha * float(q[j] @ k[j]) + wpos[0] + wtime[0]
        want = (silu(xh) * vc + silu(xs) * v[j]) / c.n
        assert np.max(np.abs(got[j, 0] - want)) <= 1e-13, (j, got[j, 0], want)


def pin_rab_cached_rows_match(lib) -> None:
    """Sampled rows equal the full output's rows."""
    cc, r, hts = _case([20, 0, 300], [40, 3, 70], 2, 128, "fp16", seed=631, npos=200)
    full = _cached(cc, r, hts, lib)
    c = cc.cand
    toks = np.array([0, 19, 39, 40, 42, 43, 100, 112], dtype=np.int64)
    hds = np.array([1, 0, 1, 0, 1, 1, 0, 1], dtype=np.int32)
    got = oracle.rows_rab_cached(c.q, c.k, c.v, c.offsets, cc.k_cache, cc.v_cache,
                                 cc.hist_offsets, r.timestamps, hts, r.pos_bias, r.time_bias,
                                 c.heads, c.d, c.alpha, c.n, c.dtype, toks, hds, lib=lib)
    assert np.array_equal(got, full[toks, hds])


RAB_CACHED_PINS = [pin_rab_cached_equals_target_aware, pin_rab_cached_zero_tables_is_cached,
                   pin_rab_cached_one_cached_key_closed_form, pin_rab_cached_rows_match]
