"""A host model of the work-item numbering the scheduler kernel builds.

The model follows the rules of schedule.hip / schedule.h: sequences ranked by
Q-tile count (largest first; input order above the sort limit), (rank, head)
pairs dealt to NQ queues in snake order, items of a sorted queue numbered
level by level from the last Q tile down (bands), items of an unsorted queue
pair by pair, and a per-queue prefix decoded by a 64-way search.  On random
jagged batches it checks that the queues together produce every
(sequence, head, Q tile) exactly once, never a tile past a sequence's end, and
that a sorted queue hands out items in non-increasing cost.
"""
import numpy as np
import pytest

NQ = 8


def queue_pair(i, x):
    return i * NQ + ((NQ - 1 - x) if (i & 1) else x)


def build(lengths, heads, bq, sort_limit=16384):
    L = np.asarray(lengths, np.int64)
    nt = (np.maximum(L, 0) + bq - 1) // bq
    N = len(L)
    bands = N <= sort_limit
    if bands:
        order = sorted(range(N), key=lambda i: (-nt[i], i))
    else:
        order = list(range(N))
    ntile = [int(nt[i]) for i in order]
    pairs = N * heads
    qlen = (pairs + NQ - 1) // NQ
    qprefix = np.zeros((NQ, qlen + 1), np.int64)
    counts = np.zeros(NQ, np.int64)
    for x in range(NQ):
        pos = [i for i in range(qlen + 1) if queue_pair(i, x) < pairs]
        n = len(pos)
        assert pos == list(range(n))
        t = [ntile[queue_pair(i, x) // heads] for i in range(n)] + [0]
        run = 0
        for i in range(n):
            qprefix[x, i] = run
            run += (t[i] - t[i + 1]) * (i + 1) if bands else t[i]
        qprefix[x, n] = run
        counts[x] = n
    return bands, order, ntile, qprefix, counts


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


def decode(bands, order, ntile, qprefix, counts, heads, x, w):
    b = search(qprefix[x], int(counts[x]), w)
    local = w - int(qprefix[x, b])
    if not bands:
        p = queue_pair(b, x)
        rank = p // heads
        return order[rank], p - rank * heads, ntile[rank] - 1 - local
    lvl, i = divmod(local, b + 1)
    p = queue_pair(i, x)
    rank = p // heads
    top = ntile[queue_pair(b, x) // heads]
    return order[rank], p - rank * heads, top - 1 - lvl


@pytest.mark.parametrize("seed", range(12))
def test_every_item_once(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 300))
    lengths = rng.integers(0, 2000, size=N)
    lengths[rng.random(N) < 0.2] = 0
    heads = int(rng.integers(1, 5))
    bq = int(rng.choice([32, 64, 128, 256]))
    limit = 16384 if seed % 3 else 10  # exercise the input-order path too
    bands, order, ntile, qprefix, counts = build(lengths, heads, bq, sort_limit=limit)
    seen = set()
    loads = []
    for x in range(NQ):
        total = int(qprefix[x, counts[x]])
        costs = []
        for w in range(total):
            i, h, j = decode(bands, order, ntile, qprefix, counts, heads, x, w)
            assert 0 <= h < heads and 0 <= j and j * bq < lengths[i]
            assert (i, h, j) not in seen
            seen.add((i, h, j))
            costs.append(j + 1)
        if bands:
            assert all(a >= b for a, b in zip(costs, costs[1:]))
        loads.append(sum(costs))
    expect = sum(int((l + bq - 1) // bq) for l in lengths) * heads
    assert len(seen) == expect


def test_search_edges():
    a = [0, 0, 0, 5, 5, 9]
    for w in range(9):
        p = search(a, 5, w)
        assert a[p] <= w < a[p + 1]
