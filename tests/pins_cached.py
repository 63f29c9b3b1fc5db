"""Pins for the oracle's cached-history form of M-FALCON.

Source: HSTU paper translation, Appendix H (the encoder-level K/V cache and
Algorithm 1's loop over micro-batches): a micro-batch computes q, k, v for its
candidates only and attends, under the target-aware mask, to the cached
history's K and V plus itself.  Each pin raises AssertionError when the
oracle disagrees with a closed form, with the equivalence the appendix states
(the cached pass gives the candidates exactly what one pass over history +
candidates gives), with the dense pair-set evaluation on the concatenated sequence,
or with separate causal passes per candidate.
"""
from __future__ import annotations

import os

import numpy as np

import oracle
import workloads
from pins import _eval, _parse_tokens

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "falcon_cached_hand_worked.txt")


def cached_golden_cases(path: str = GOLDEN):
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
        coff = np.array([int(x) for x in c["cand_offsets"].split()], dtype=np.int32)
        hoff = np.array([int(x) for x in c["hist_offsets"].split()], dtype=np.int32)
        arr = {name: _parse_tokens(c[name], heads, d, float) for name in ("q", "k", "v", "kc", "vc")}
        out.append(dict(name=c["name"], heads=heads, d=d, coff=coff, hoff=hoff,
                        alpha=float(c["alpha"]), n=float(c["n"]),
                        expect=_parse_tokens(c["expect"], heads, d, _eval), **arr))
    return out


def random_cached(hist, cand, heads, d, dtype, seed, alpha=None, n=None):
    """A cached-history problem: per request, a history case (kc, vc) and a
    candidate case (q, k, v), all i.i.d. normal."""
    hc = workloads.make_case(hist, heads, d, dtype, seed=seed, alpha=alpha, n=n)
    cc = workloads.make_case(cand, heads, d, dtype, seed=seed + 1, alpha=alpha, n=n)
    return hc, cc


def concatenated(hc, cc):
    """Per request: history rows then candidate rows (the sequence Algorithm 1
    feeds to one pass), its offsets, and the candidate count per request.  The
    history's queries are zero (their outputs are not compared)."""
    qs, ks, vs, lens = [], [], [], []
    for i in range(hc.num_seqs):
        ha, hb = int(hc.offsets[i]), int(hc.offsets[i + 1])
        ca, cb = int(cc.offsets[i]), int(cc.offsets[i + 1])
        qs += [np.zeros_like(hc.k[ha:hb]), cc.q[ca:cb]]
        ks += [hc.k[ha:hb], cc.k[ca:cb]]
        vs += [hc.v[ha:hb], cc.v[ca:cb]]
        lens.append((hb - ha) + (cb - ca))
    return (np.concatenate(qs), np.concatenate(ks), np.concatenate(vs),
            workloads.offsets_from_lengths(lens), np.diff(cc.offsets).astype(np.int32))


def cand_rows_of_concat(hc, cc, full):
    """The candidate rows of an output over the concatenated sequences."""
    off = workloads.offsets_from_lengths(np.diff(hc.offsets) + np.diff(cc.offsets))
    rows = []
    for i in range(hc.num_seqs):
        h = int(hc.offsets[i + 1] - hc.offsets[i])
        rows.append(full[int(off[i]) + h:int(off[i + 1])])
    return np.concatenate(rows)


def cached_of(hc, cc, dtype, lib):
    return oracle.fwd_cached(cc.q, cc.k, cc.v, cc.offsets, hc.k, hc.v, hc.offsets, cc.heads,
                             cc.d, cc.alpha, cc.n, dtype, lib=lib)


def pin_cached_hand_worked(lib) -> None:
    """Closed-form cases, every storage type (inputs are small integers)."""
    for c in cached_golden_cases():
        for dtype in ("fp32", "fp16", "bf16"):
            q, k, v, kc, vc = (workloads.cast_values(c[x].astype(np.float32), dtype)
                               for x in ("q", "k", "v", "kc", "vc"))
            got = oracle.fwd_cached(q, k, v, c["coff"], kc, vc, c["hoff"], c["heads"], c["d"],
                                    c["alpha"], c["n"], dtype, lib=lib)
            err = float(np.max(np.abs(got - c["expect"])))
            assert err <= 1e-13 * max(1.0, float(np.max(np.abs(c["expect"])))), \
                (c["name"], dtype, got.ravel(), c["expect"].ravel())


def pin_cached_equals_one_pass(lib) -> None:
    """Appendix H: with the history's K and V taken from the cache, a
    micro-batch's candidates get what one pass over history + candidates under
    the target-aware mask gives them (here: the row loop with the mask, and the
    dense pair-set evaluation with its visibility matrix)."""
    hc, cc = random_cached([7, 0, 40, 3], [3, 2, 5, 0], 2, 64, "bf16", seed=61, n=40.0)
    got = cached_of(hc, cc, "bf16", lib)
    q, k, v, off, tg = concatenated(hc, cc)
    loop = oracle.fwd(q, k, v, off, 2, 64, cc.alpha, cc.n, "bf16", lib=lib, num_targets=tg)
    dense = oracle.dense_pairs(q, k, v, off, 2, 64, cc.alpha, cc.n, "bf16", num_targets=tg)
    for ref in (cand_rows_of_concat(hc, cc, loop), cand_rows_of_concat(hc, cc, dense)):
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))


def pin_cached_equals_separate_causal(lib) -> None:
    """Each candidate's row is the last row of a plain causal pass over the
    history followed by that candidate alone."""
    hc, cc = random_cached([9, 4], [4, 3], 2, 64, "fp32", seed=71)
    got = cached_of(hc, cc, "fp32", lib)
    m = 0
    for i in range(hc.num_seqs):
        ha, hb = int(hc.offsets[i]), int(hc.offsets[i + 1])
        for r in range(int(cc.offsets[i]), int(cc.offsets[i + 1])):
            q = np.concatenate([np.zeros_like(hc.q[ha:hb]), cc.q[r:r + 1]])
            k = np.concatenate([hc.k[ha:hb], cc.k[r:r + 1]])
            v = np.concatenate([hc.v[ha:hb], cc.v[r:r + 1]])
            one = oracle.fwd(q, k, v, [0, hb - ha + 1], 2, 64, cc.alpha, cc.n, "fp32", lib=lib)
            assert np.allclose(got[r], one[hb - ha], rtol=0, atol=1e-14), (i, r)
            m += 1
    assert m == 7


def pin_cached_without_history(lib) -> None:
    """No history: each candidate sees only itself, out = silu(alpha <q, k>) v / n
    (numpy, per row)."""
    hc, cc = random_cached([0, 0], [5, 2], 3, 64, "fp16", seed=81, n=3.0)
    got = cached_of(hc, cc, "fp16", lib)
    q, k, v = (oracle.widen(a, "fp16") for a in (cc.q, cc.k, cc.v))
    x = cc.alpha * np.sum(q * k, axis=-1, keepdims=True)
    ref = x / (1.0 + np.exp(-x)) * v / cc.n
    assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, float(np.max(np.abs(ref))))


def pin_cached_rows_match(lib) -> None:
    """Sampled rows equal the full output's rows."""
    hc, cc = random_cached([6, 11, 2], [3, 4, 2], 2, 128, "bf16", seed=91)
    full = cached_of(hc, cc, "bf16", lib)
    toks = np.array([0, 2, 3, 6, 7, 8], dtype=np.int64)
    hds = np.array([0, 1, 1, 0, 1, 0], dtype=np.int32)
    r = oracle.rows_cached(cc.q, cc.k, cc.v, cc.offsets, hc.k, hc.v, hc.offsets, 2, 128,
                           cc.alpha, cc.n, "bf16", toks, hds, lib=lib)
    assert np.array_equal(r, full[toks, hds])


CACHED_PINS = [pin_cached_hand_worked, pin_cached_equals_one_pass,
               pin_cached_equals_separate_causal, pin_cached_without_history,
               pin_cached_rows_match]
