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
__device__ inline Item decode_item(const WorkList& wl, int num_seqs, int heads, int x, int w) {
    const int pairs = num_seqs * heads;
    const int* pre = wl.qprefix + x * (wl.qlen + 1);
    const int b = wave_search(pre, queue_pairs(pairs, x), w);   // band (or pair)
    const int local = w - pre[b];
    if (wl.ctl[CTL_MODE] == QUEUE_PAIRS) {
        const int p = queue_pair(b, x);
        const int rank = p / heads;
        Item it;
        it.head = p - rank * heads;
        it.qtile = wl.ntile[rank] - 1 - local;
        it.seq = wl.order[rank];
        return it;
    }
    const int per_level = b + 1;                                 // pairs taking part
    const int lvl = local / per_level;
    const int i = local - lvl * per_level;                       // pair position in queue
    const int p = queue_pair(i, x);
    const int rank = p / heads;
    const int top = wl.ntile[queue_pair(b, x) / heads];          // tiles of the band's last pair
    Item it;
    it.head = p - rank * heads;
    it.qtile = top - 1 - lvl;
    it.seq = wl.order[rank];
    return it;
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
    __device__ ItemSource() : queue(current_xcd() % NQ) {}

    // Returns false when every queue is empty.  On true, *x and *w name the item.
    __device__ bool next(const WorkList& wl, int* slot, int* x, int* w) {
        for (;;) {
            if (threadIdx.x == 0) slot[0] = atomicAdd(wl.ctl + CTL_NEXT + CTL_LINE * queue, 1);
            __syncthreads();
            const int got = __builtin_amdgcn_readfirstlane(slot[0]);
            __syncthreads();
            if (got < wl.ctl[CTL_TOTAL + queue]) {
                *x = queue;
                *w = got;
                return true;
            }
            if (threadIdx.x < NQ) {
                const int q = threadIdx.x;
                const int taken = __hip_atomic_load(wl.ctl + CTL_NEXT + CTL_LINE * q,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                slot[q] = wl.ctl[CTL_TOTAL + q] - taken;
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

}  // namespace hstu
