// Device-side work distribution: queue selection, item fetch and decoding of
// an item number into (sequence, head, Q tile).
//
// The Ascend HSTU blog ("都是生成式推荐，为什么昇腾这么快？", §3.2) classifies
// each (Q block, K block) pair as all-ones, lower-triangular or all-zero and
// skips the all-zero ones; §4.2 computes only the real tokens of a jagged
// batch.  Here a work item is one Q tile of one (sequence, head); tile pairs
// above the diagonal are never enumerated, and Q tiles exist only for real
// tokens.  The HSTU paper translation (§3.2) views the ragged attention as a
// grouped GEMM of differently sized problems; sequences are ranked longest
// first so the pool of persistent workgroups ends on short items.
#pragma once

#include "internal.h"

namespace hstu {

struct Item {
    int seq;
    int head;
    int qtile;
};

// Largest p in [0, n) with a[p] <= w, given a non-decreasing a with
// a[0] <= w < a[n].  All 64 lanes of the wave probe together, so each round
// shrinks the range 64-fold; the result is wave-uniform.
__device__ inline int wave_search(const int* __restrict__ a, int n, int w) {
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int len = hi - lo;
        const int stride = (len + 63) >> 6;
        const int p = lo + (lane + 1) * stride;
        const bool ok = (p < hi) && (a[p] <= w);
        const unsigned long long m = __ballot(ok);
        const int c = __popcll(m);
        lo += c * stride;
        hi = min(hi, lo + stride);
    }
    return lo;
}

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ inline int current_xcd() {
    return (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 15u);
}

// Pairs in queue x when there are `pairs` (rank, head) pairs in total: every
// full round gives each queue one pair; the last, partial round gives its
// first pairs % NQ positions (which queues those are depends on the round's
// direction).
__device__ inline int queue_pairs(int pairs, int x) {
    const int full = pairs / NQ, rem = pairs % NQ;
    const int pos = (full & 1) ? NQ - 1 - x : x;  // x's position in the last round
    return full + (pos < rem ? 1 : 0);
}

// Item w of queue x.
__device__ inline Item decode_item(const Tables& tb, int num_seqs, int heads, int x, int w) {
    const int pairs = num_seqs * heads;
    const int* pre = tb.qprefix + x * (tb.qlen + 1);
    const int b = wave_search(pre, queue_pairs(pairs, x), w);   // band (or pair)
    const int local = w - pre[b];
    if (tb.mode == QUEUE_PAIRS) {
        const int p = queue_pair(b, x);
        const int rank = p / heads;
        Item it;
        it.head = p - rank * heads;
        it.qtile = tb.ntile[rank] - 1 - local;
        it.seq = tb.order[rank];
        return it;
    }
    const int per_level = b + 1;                                 // pairs taking part
    const int lvl = local / per_level;
    const int i = local - lvl * per_level;                       // pair position in queue
    const int p = queue_pair(i, x);
    const int rank = p / heads;
    const int top = tb.ntile[queue_pair(b, x) / heads];          // tiles of the band's last pair
    Item it;
    it.head = p - rank * heads;
    it.qtile = top - 1 - lvl;
    it.seq = tb.order[rank];
    return it;
}

// The global work list as tables.
__device__ inline Tables global_tables(const WorkList& wl) {
    Tables tb;
    tb.order = wl.order;
    tb.ntile = wl.ntile;
    tb.qprefix = wl.qprefix;
    tb.totals = wl.ctl + CTL_TOTAL;
    tb.qlen = wl.qlen;
    tb.mode = wl.ctl[CTL_MODE];
    return tb;
}

// Builds the queue tables of a fused launch in LDS, with every thread of the
// workgroup (blockDim.x >= FUSE_SEQS, a multiple of 64).  The same ranking and
// numbering as the work-list kernel: sequences by Q-tile count, largest first
// (ties by index), pairs dealt to the queues in snake order, per queue the
// first item of each band (or of each pair, when no sequence has more than
// PAIRS_MAX_TILES tiles).  Workgroup 0 publishes the offset flags.
__device__ inline Tables build_local_tables(LocalTables& lt, int* scratch, const int32_t* off,
                                            int num_seqs, int heads, int bq, int* ctl) {
    const int tid = threadIdx.x;
    int* t_in = scratch;                 // [FUSE_SEQS] tile count by sequence id
    if (tid == 0) lt.flags = 0;
    __syncthreads();
    if (tid < num_seqs) {
        long long s = (long long)off[tid + 1] - (long long)off[tid];
        int fl = 0;
        if (tid == 0 && off[0] != 0) fl |= 1;
        if (s < 0) {
            fl |= 2;
            s = 0;
        }
        t_in[tid] = (int)((s + bq - 1) / bq);
        if (fl) atomicOr(&lt.flags, fl);
    }
    __syncthreads();
    // Rank: sequences with more tiles, then equal tiles and a smaller index.
    if (tid < num_seqs) {
        const int t = t_in[tid];
        int rank = 0;
        for (int j = 0; j < num_seqs; ++j) {
            const int u = t_in[j];
            rank += (u > t) || (u == t && j < tid);
        }
        lt.order[rank] = tid;
        lt.ntile[rank] = t;
    }
    __syncthreads();
    // Band (or pair) prefix: threads 32x .. 32x+31 scan queue x, CHUNK
    // positions each.  (ntile[0]: the largest tile count)
    const int mode = lt.ntile[0] <= PAIRS_MAX_TILES ? QUEUE_PAIRS : QUEUE_BANDS;
    const int pairs = num_seqs * heads;
    const int qlen = (pairs + NQ - 1) / NQ;
    const int full = pairs / NQ, rem = pairs % NQ;
    auto position_exists = [&](int i, int x) {
        if (i < full) return true;
        if (i > full) return false;
        const int pos = (full & 1) ? NQ - 1 - x : x;
        return pos < rem;
    };
    constexpr int CHUNK = (FUSE_QLEN + 31) / 32;
    if (tid < 32 * NQ) {
        const int x = tid >> 5, l = tid & 31;
        long long term[CHUNK];
        long long sum = 0;
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) {
            const int i = l * CHUNK + c;
            long long v = 0;
            if (position_exists(i, x)) {
                const long long ti = lt.ntile[queue_pair(i, x) / heads];
                const long long tn =
                        position_exists(i + 1, x) ? lt.ntile[queue_pair(i + 1, x) / heads] : 0;
                v = mode == QUEUE_PAIRS ? ti : (ti - tn) * (i + 1);
            }
            term[c] = v;
            sum += v;
        }
        long long inc = sum;   // inclusive scan of the chunk sums over the 32 threads
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            const long long y = __shfl_up(inc, o, 32);
            if (l >= o) inc += y;
        }
        long long run = inc - sum;
#pragma unroll
        for (int c = 0; c < CHUNK; ++c) {
            const int i = l * CHUNK + c;
            if (position_exists(i, x)) lt.qprefix[x * (qlen + 1) + i] = (int)min(run, 0x7fffffffLL);
            run += term[c];
        }
        if (l == 31) {
            const int pos = (full & 1) ? NQ - 1 - x : x;
            const int nx = full + (pos < rem ? 1 : 0);
            int total = (int)inc;
            if (inc > 0x7fffffffLL) {   // refuse to run rather than wrap
                atomicOr(&lt.flags, 4);
                total = 0;
            }
            lt.qprefix[x * (qlen + 1) + nx] = total;
            lt.totals[x] = total;
        }
    }
    __syncthreads();
    if (blockIdx.x == 0 && tid == 0) {
        ctl[CTL_FLAGS] = lt.flags;
        ctl[CTL_MODE] = mode;
    }
    Tables tb;
    tb.order = lt.order;
    tb.ntile = lt.ntile;
    tb.qprefix = lt.qprefix;
    tb.totals = lt.totals;
    tb.qlen = qlen;
    tb.mode = mode;
    return tb;
}

// Hands out items to a workgroup: its own XCD's queue first, then, once that
// one is empty, the queue with the most items left.  Thread 0 takes an item
// with an atomic and shares it through LDS; when the queue it drew from is
// found empty, threads 0..NQ-1 read every queue's counter at once (one round
// trip instead of one atomic per queue), so a workgroup that runs out of work
// learns it in two round trips.  The caller passes NQ ints of LDS and calls
// next() from every thread.
struct ItemSource {
    int queue;   // queue currently being drained
    int* next_;  // this call's counter set
    __device__ ItemSource(int* ctl, int set)
        : queue(current_xcd() % NQ), next_(ctl + CTL_NEXT + CTL_LINE * NQ * set) {}

    // Returns false when every queue is empty.  On true, *x and *w name the item.
    __device__ bool next(const Tables& tb, int* slot, int* x, int* w) {
        for (;;) {
            if (threadIdx.x == 0) slot[0] = atomicAdd(next_ + CTL_LINE * queue, 1);
            __syncthreads();
            const int got = __builtin_amdgcn_readfirstlane(slot[0]);
            __syncthreads();
            if (got < tb.totals[queue]) {
                *x = queue;
                *w = got;
                return true;
            }
            if (threadIdx.x < NQ) {
                const int q = threadIdx.x;
                const int taken = __hip_atomic_load(next_ + CTL_LINE * q,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                slot[q] = tb.totals[q] - taken;
            }
            __syncthreads();
            int best = -1, most = 0;
#pragma unroll
            for (int i = 1; i <= NQ; ++i) {
                const int q = (queue + i) % NQ;
                const int left = slot[q];
                if (left > most) {
                    most = left;
                    best = q;
                }
            }
            __syncthreads();
            if (best < 0) return false;
            queue = __builtin_amdgcn_readfirstlane(best);
        }
    }
};

// Clears counter sets first .. first + count - 1 (mod NSETS): the sets the
// next call on this work list will use, none of which this launch touches.
// Called by every thread; workgroup 0's first NQ * count threads do it.
__device__ inline void clear_sets(int* ctl, int first, int count) {
    const int t = threadIdx.x;
    if (blockIdx.x == 0 && t < NQ * count) {
        const int set = (first + t / NQ) % NSETS;
        __hip_atomic_store(ctl + CTL_NEXT + CTL_LINE * (NQ * set + t % NQ), 0, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace hstu
