"""A host model of the work-item numbering the scheduler kernel builds.

The model follows the same rules as schedule.hip / schedule.h (sorted bands,
or input order above the sort limit) and checks, on random jagged batches,
that every (sequence, head, Q tile) is produced exactly once, that no tile
above the causal diagonal or past a sequence's end is produced, and that band
order hands out items in non-increasing cost.
"""
import numpy as np
import pytest


def build(lengths, heads, bq, sort_limit=16384):
    L = np.asarray(lengths, np.int64)
    nt = (np.maximum(L, 0) + bq - 1) // bq
    N = len(L)
    if N <= sort_limit:
        order = sorted(range(N), key=lambda i: (-nt[i], i))
        ntile = [int(nt[i]) for i in order] + [0]
        terms = [(ntile[m] - ntile[m + 1]) * (m + 1) * heads for m in range(N)]
        mode = "bands"
    else:
        order = list(range(N))
        ntile = [int(x) for x in nt] + [0]
        terms = [ntile[i] * heads for i in range(N)]
        mode = "seqs"
    prefix = np.concatenate([[0], np.cumsum(terms)]).astype(np.int64)
    return mode, order, ntile, prefix


def search(a, n, w):
    """The wave search: 64 probes per round."""
    lo, hi = 0, n
    while hi - lo > 1:
        length = hi - lo
        stride = (length + 63) >> 6
        c = 0
        for lane in range(64):
            p = lo + (lane + 1) * stride
            if p < hi and a[p] <= w:
                c += 1
        lo += c * stride
        hi = min(hi, lo + stride)
    return lo


def decode(mode, order, ntile, prefix, N, heads, w):
    m = search(prefix, N, w)
    local = w - prefix[m]
    if mode == "bands":
        per = (m + 1) * heads
        lvl, rem = divmod(local, per)
        rank, h = divmod(rem, heads)
        return order[rank], h, ntile[m] - 1 - lvl
    lvl, h = divmod(local, heads)
    return m, h, ntile[m] - 1 - lvl


@pytest.mark.parametrize("seed", range(12))
def test_every_item_once(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 300))
    lengths = rng.integers(0, 2000, size=N)
    lengths[rng.random(N) < 0.2] = 0
    heads = int(rng.integers(1, 5))
    bq = int(rng.choice([32, 64, 128]))
    limit = 16384 if seed % 3 else 10  # exercise both modes
    mode, order, ntile, prefix = build(lengths, heads, bq, sort_limit=limit)
    total = int(prefix[-1])
    seen = set()
    costs = []
    for w in range(total):
        i, h, j = decode(mode, order, ntile, prefix, N, heads, w)
        assert 0 <= h < heads and 0 <= j and j * bq < lengths[i]
        assert (i, h, j) not in seen
        seen.add((i, h, j))
        costs.append(j)
    expect = sum(int((l + bq - 1) // bq) for l in lengths) * heads
    assert len(seen) == expect == total
    if mode == "bands":
        assert all(a >= b for a, b in zip(costs, costs[1:]))


def test_search_edges():
    a = [0, 0, 0, 5, 5, 9]
    for w in range(9):
        p = search(a, 5, w)
        assert a[p] <= w < a[p + 1]
