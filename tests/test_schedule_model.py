"""A host model of the work-item numbering the scheduler kernel builds.

The model follows the rules of schedule.hip / schedule.h: sequences ranked by
Q-tile count (largest first; input order above the sort limit), (rank, head)
pairs dealt to NQ queues in snake order, items of a sorted queue numbered
level by level from the last Q tile down (bands), items of an unsorted queue,
or of any queue when no sequence has more than PAIRS_MAX_TILES tiles, pair by
pair, and a per-queue prefix decoded by a 64-way search.  On random
jagged batches it checks that the queues together produce every
(sequence, head, Q tile) exactly once, never a tile past a sequence's end, and
that a sorted queue hands out items in non-increasing cost.
"""
import numpy as np
import pytest

NQ = 8
PAIRS_MAX_TILES = 2


def queue_pair(i, x):
    return i * NQ + ((NQ - 1 - x) if (i & 1) else x)


def build(lengths, heads, bq, sort_limit=16384):
    L = np.asarray(lengths, np.int64)
    nt = (np.maximum(L, 0) + bq - 1) // bq
    N = len(L)
    sort = N <= sort_limit
    bands = sort and N > 0 and int(nt.max()) > PAIRS_MAX_TILES
    if sort:
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
    if seed % 4 == 3:   # short sequences only: pair order on sorted ranks
        lengths = np.minimum(lengths, 2 * bq)
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


# ---------------------------------------------------------------------------
# The tables a small-batch launch builds inside the attention kernel
# (build_local_tables in schedule.h): rank by an all-pairs count, then per
# queue 32 threads scan CHUNK consecutive band terms each.  Emulated step by
# step here and checked against the model above.
FUSE_SEQS, FUSE_PAIRS = 256, 2048
FUSE_QLEN = FUSE_PAIRS // NQ
CHUNK = (FUSE_QLEN + 31) // 32


def build_local(lengths, heads, bq):
    L = np.asarray(lengths, np.int64)
    n = len(L)
    t_in = [int((max(int(s), 0) + bq - 1) // bq) for s in L]
    order = [0] * n
    ntile = [0] * n
    for tid in range(n):
        t = t_in[tid]
        rank = sum(1 for j in range(n) if t_in[j] > t or (t_in[j] == t and j < tid))
        order[rank] = tid
        ntile[rank] = t
    pairs = n * heads
    qlen = (pairs + NQ - 1) // NQ
    full, rem = pairs // NQ, pairs % NQ
    bands = ntile[0] > PAIRS_MAX_TILES

    def exists(i, x):
        if i < full:
            return True
        if i > full:
            return False
        pos = (NQ - 1 - x) if (full & 1) else x
        return pos < rem

    qprefix = np.full((NQ, qlen + 1), -1, np.int64)
    totals = [0] * NQ
    for x in range(NQ):
        sums, terms = [], []
        for l in range(32):
            tl = []
            for c in range(CHUNK):
                i = l * CHUNK + c
                v = 0
                if exists(i, x):
                    ti = ntile[queue_pair(i, x) // heads]
                    tn = ntile[queue_pair(i + 1, x) // heads] if exists(i + 1, x) else 0
                    v = (ti - tn) * (i + 1) if bands else ti
                tl.append(v)
            terms.append(tl)
            sums.append(sum(tl))
        inc = np.cumsum(sums)
        for l in range(32):
            run = int(inc[l] - sums[l])
            for c in range(CHUNK):
                i = l * CHUNK + c
                if exists(i, x):
                    qprefix[x, i] = run
                run += terms[l][c]
        pos = (NQ - 1 - x) if (full & 1) else x
        nx = full + (1 if pos < rem else 0)
        qprefix[x, nx] = int(inc[31])
        totals[x] = int(inc[31])
    return bands, order, ntile, qprefix, totals


@pytest.mark.parametrize("seed", range(10))
def test_local_tables_match_model(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, FUSE_SEQS + 1))
    heads = int(rng.integers(1, FUSE_PAIRS // N + 1))
    heads = min(heads, 16)
    lengths = rng.integers(0, 3000, size=N)
    lengths[rng.random(N) < 0.2] = 0
    bq = int(rng.choice([32, 128, 256]))
    if seed % 3 == 2:   # short sequences only: pair order
        lengths = np.minimum(lengths, 2 * bq)
    l_bands, order, ntile, qprefix, totals = build_local(lengths, heads, bq)
    bands, m_order, m_ntile, m_qprefix, counts = build(lengths, heads, bq)
    assert l_bands == bands and order == m_order and ntile == m_ntile
    for x in range(NQ):
        n = int(counts[x])
        assert list(qprefix[x, :n + 1]) == list(m_qprefix[x, :n + 1])
        assert totals[x] == int(m_qprefix[x, n])
    # and every item decodes to a real tile, once
    seen = set()
    for x in range(NQ):
        for w in range(totals[x]):
            i, h, j = decode(bands, order, ntile, qprefix, counts, heads, x, w)
            assert 0 <= h < heads and 0 <= j and j * bq < lengths[i]
            seen.add((i, h, j))
    assert len(seen) == sum(int((l + bq - 1) // bq) for l in lengths) * heads
