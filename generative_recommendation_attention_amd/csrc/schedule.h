// Device-side decoding of a work-item number into (sequence, head, Q tile).
//
// The Ascend HSTU blog ("都是生成式推荐，为什么昇腾这么快？", §3.2) classifies
// each (Q block, K block) pair as all-ones, lower-triangular or all-zero and
// skips the all-zero ones; §4.2 computes only the real tokens of a jagged
// batch.  Here a work item is one Q tile of one (sequence, head); the tile
// pairs above the diagonal are never enumerated, and a Q tile exists only for
// real tokens.  The HSTU paper translation (§3.2) views the ragged attention
// as a grouped GEMM of differently sized problems; items are ordered longest
// first so that a pool of persistent workgroups ends with short ones.
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

__device__ inline Item decode_item(const WorkList& wl, int mode, int num_seqs, int heads, int w) {
    Item it;
    const int m = wave_search(wl.prefix, num_seqs, w);
    const int local = w - wl.prefix[m];
    if (mode == MODE_BANDS) {
        // Band m: levels ntile[m+1] .. ntile[m]-1, ranks 0..m take part.
        const int per_level = (m + 1) * heads;
        const int lvl = local / per_level;
        const int rem = local - lvl * per_level;
        const int rank = rem / heads;
        it.head = rem - rank * heads;
        it.qtile = wl.ntile[m] - 1 - lvl;
        it.seq = wl.order[rank];
    } else {
        const int lvl = local / heads;
        it.head = local - lvl * heads;
        it.qtile = wl.ntile[m] - 1 - lvl;
        it.seq = m;
    }
    return it;
}

}  // namespace hstu
