// Work-list build: one workgroup turns the jagged offsets into the queues the
// attention kernel drains (see schedule.h and internal.h).
//
// 1. Rank the sequences by Q-tile count, largest first: a counting sort (LDS
//    histogram + scatter) when the largest count fits the histogram, else an
//    LDS bitonic sort; above SORT_MAX sequences, input order.
// 2. Deal the (rank, head) pairs to the NQ queues in snake order and scan,
//    per queue, the item count of each band into qprefix.
// 3. Reset the item counters of both counter sets, so a forward call needs no
//    memset (the attention kernel clears the set of the call after it, for
//    launches that build their tables themselves).
#include <hip/hip_ext.h>

#include "internal.h"

namespace hstu {

namespace {

constexpr int SCHED_THREADS = 1024;
constexpr int SCHED_WAVES = SCHED_THREADS / 64;
constexpr int HIST_MAX = 8192;  // tile-count values the counting sort handles
constexpr int CACHE = 4;        // tile counts each thread keeps in registers

enum : int { RANK_COUNTING = 0, RANK_BITONIC = 1, RANK_INPUT = 2 };

struct SchedShared {
    long long wave_sum[SCHED_WAVES][NQ];
    long long carry[NQ];
    int flags;
    int max_tiles;
};

// Inclusive scan over threads of one value per thread, segmented by
// thread % seg (seg = 1: a plain scan; seg = NQ: one scan per queue, since the
// thread index and the pair index agree mod NQ).  Returns the thread's
// inclusive prefix within its segment.  Callers separate two calls with a
// barrier.
__device__ long long segmented_scan(long long v, int seg, SchedShared& sh) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int off = seg; off < 64; off <<= 1) {
        const long long y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    // The wave's last `seg` lanes hold its per-segment totals.
    if (lane >= 64 - seg) sh.wave_sum[wave][lane % seg] = v;
    __syncthreads();
    if (tid < seg) {
        long long run = 0;
        for (int w = 0; w < SCHED_WAVES; ++w) {
            const long long t = sh.wave_sum[w][tid];
            sh.wave_sum[w][tid] = run;
            run += t;
        }
    }
    __syncthreads();
    return v + sh.wave_sum[wave][lane % seg];
}

// counters[t] += 1 for every active lane of the wave, with one LDS atomic
// per distinct t in the wave instead of one per lane (a batch of short
// sequences has only a few tile counts, and per-lane atomics on those few
// addresses serialise).  Returns the lane's slot: the counter's old value
// plus the lane's rank among the wave's lanes with the same t.  Called by
// every lane of the wave.
__device__ inline int wave_counted_add(int* counters, int t, bool active) {
    const int lane = threadIdx.x & 63;
    unsigned long long pending = __ballot(active);
    int slot = 0;
    while (pending) {
        const int leader = __builtin_ctzll(pending);
        const int v = __builtin_amdgcn_readlane(t, leader);
        const unsigned long long same = __ballot(active && t == v);
        int base = 0;
        if (lane == leader) base = atomicAdd(&counters[v], __popcll(same));
        base = __builtin_amdgcn_readlane(base, leader);
        if (active && t == v) slot = base + __popcll(same & ((1ull << lane) - 1ull));
        pending &= ~same;
    }
    return slot;
}

__global__ __launch_bounds__(SCHED_THREADS) void schedule_kernel(
        const int32_t* __restrict__ off, int num_seqs, int heads, int bq, WorkList wl,
        int force_kind) {
    extern __shared__ unsigned long long dyn[];
    __shared__ SchedShared sh;
    const int tid = threadIdx.x;
    if (tid < NQ) sh.carry[tid] = 0;
    if (tid == 0) {
        sh.flags = 0;
        sh.max_tiles = 0;
    }
    __syncthreads();

    int flags = 0;
    if (tid == 0 && num_seqs > 0 && off[0] != 0) flags |= 1;
    auto tiles_of = [&](int i) -> int {
        long long s = (long long)off[i + 1] - (long long)off[i];
        if (s < 0) {
            flags |= 2;
            s = 0;
        }
        return (int)((s + bq - 1) / bq);
    };

    // Each thread's first CACHE sequences (i = tid + k * SCHED_THREADS) keep
    // their tile count in registers, so the offsets are read from memory once
    // for batches of up to SCHED_THREADS * CACHE sequences.
    int tcache[CACHE];
#pragma unroll
    for (int k = 0; k < CACHE; ++k) {
        const int i = tid + k * SCHED_THREADS;
        tcache[k] = i < num_seqs ? tiles_of(i) : 0;
    }
    // f(i, tiles of i) for this thread's sequences.
    auto for_each_seq = [&](auto f) {
#pragma unroll
        for (int k = 0; k < CACHE; ++k) {
            const int i = tid + k * SCHED_THREADS;
            if (i < num_seqs) f(i, tcache[k]);
        }
        for (int i = tid + CACHE * SCHED_THREADS; i < num_seqs; i += SCHED_THREADS) f(i, tiles_of(i));
    };
    // f(i, tiles of i, i < num_seqs) on every lane, with the wave converged.
    auto for_each_lane = [&](auto f) {
#pragma unroll
        for (int k = 0; k < CACHE; ++k) {
            const int i = tid + k * SCHED_THREADS;
            f(i, tcache[k], i < num_seqs);
        }
        for (int base = CACHE * SCHED_THREADS; base < num_seqs; base += SCHED_THREADS) {
            const int i = base + tid;
            const bool active = i < num_seqs;
            f(i, active ? tiles_of(i) : 0, active);
        }
    };

    // ---- 1. ranking -------------------------------------------------------
    int my_max = 0;
    for_each_seq([&](int, int t) { my_max = max(my_max, t); });
    atomicMax(&sh.max_tiles, my_max);
    __syncthreads();
    const int maxT = sh.max_tiles;
    int kind = force_kind;
    if (kind == RANK_COUNTING && maxT >= HIST_MAX) kind = RANK_BITONIC;
    if (num_seqs > SORT_MAX) kind = RANK_INPUT;

    // LDS layout: counting = hist[HIST_MAX] | cursor[HIST_MAX] | sorted[SORT_MAX] (ints);
    //             bitonic  = keys[pow2 >= num_seqs] (u64).
    int* hist = reinterpret_cast<int*>(dyn);
    int* cursor = hist + HIST_MAX;
    int* sorted = cursor + HIST_MAX;
    unsigned long long* keys = dyn;

    if (kind == RANK_COUNTING) {
        for (int v = tid; v <= maxT; v += SCHED_THREADS) hist[v] = 0;
        __syncthreads();
        for_each_lane([&](int, int t, bool active) { wave_counted_add(hist, t, active); });
        __syncthreads();
        // cursor[v] = number of sequences with more than v tiles (scan over v descending).
        for (int base = 0; base <= maxT; base += SCHED_THREADS) {
            const int v = maxT - (base + tid);
            const long long h = (v >= 0) ? hist[v] : 0;
            const long long inc = segmented_scan(h, 1, sh);
            if (v >= 0) cursor[v] = (int)(sh.carry[0] + inc - h);
            __syncthreads();
            if (tid == SCHED_THREADS - 1) sh.carry[0] += inc;
            __syncthreads();
        }
        for_each_lane([&](int i, int t, bool active) {
            const int pos = wave_counted_add(cursor, t, active);
            if (active) {
                wl.order[pos] = i;
                wl.ntile[pos] = t;
                sorted[pos] = t;
            }
        });
    } else if (kind == RANK_BITONIC) {
        int P = 1;
        while (P < num_seqs) P <<= 1;
        for (int i = tid; i < P; i += SCHED_THREADS) keys[i] = 0;
        __syncthreads();
        for_each_seq([&](int i, int t) {
            keys[i] = ((unsigned long long)(unsigned)t << 32) | (unsigned long long)(~(unsigned)i);
        });
        __syncthreads();
        for (int kk = 2; kk <= P; kk <<= 1) {
            for (int j = kk >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < P; i += SCHED_THREADS) {
                    const int ixj = i ^ j;
                    if (ixj > i) {
                        const unsigned long long a = keys[i], b = keys[ixj];
                        const bool desc = (i & kk) == 0;
                        if (desc ? (a < b) : (a > b)) {
                            keys[i] = b;
                            keys[ixj] = a;
                        }
                    }
                }
                __syncthreads();
            }
        }
        for (int m = tid; m < num_seqs; m += SCHED_THREADS) {
            wl.order[m] = (int)(~(unsigned)(keys[m] & 0xffffffffull));
            wl.ntile[m] = (int)(keys[m] >> 32);
        }
    } else {
        for_each_seq([&](int i, int t) {
            wl.order[i] = i;
            wl.ntile[i] = t;
        });
    }
    __syncthreads();
    if (tid < NQ) sh.carry[tid] = 0;
    __syncthreads();
    auto tiles_at_rank = [&](int m) -> int {
        if (kind == RANK_COUNTING) return sorted[m];
        if (kind == RANK_BITONIC) return (int)(keys[m] >> 32);
        return tiles_of(m);
    };
    const int mode = (kind == RANK_INPUT || maxT <= PAIRS_MAX_TILES) ? QUEUE_PAIRS : QUEUE_BANDS;

    // ---- 2. per-queue band prefix --------------------------------------------
    // Thread t of a chunk takes queue x = t % NQ, position i = (base + t) / NQ.
    // Band i of queue x spans levels [tiles of position i+1, tiles of position i)
    // with i + 1 pairs, so its item count is (t_i - t_{i+1}) * (i + 1).
    const int pairs = num_seqs * heads;
    const int row = wl.qlen + 1;
    const int full = pairs / NQ, rem = pairs % NQ;
    auto position_exists = [&](int i, int x) {
        if (i < full) return true;
        if (i > full) return false;
        const int pos = (full & 1) ? NQ - 1 - x : x;
        return pos < rem;
    };
    for (int base = 0; base < pairs + NQ; base += SCHED_THREADS) {
        const int x = tid % NQ;
        const int i = (base + tid) / NQ;
        long long term = 0;
        const bool here = position_exists(i, x);
        if (here) {
            const long long ti = tiles_at_rank(queue_pair(i, x) / heads);
            const long long tn = position_exists(i + 1, x) ? tiles_at_rank(queue_pair(i + 1, x) / heads) : 0;
            term = (mode == QUEUE_PAIRS) ? ti : (ti - tn) * (long long)(i + 1);
        }
        const long long inc = segmented_scan(term, NQ, sh);
        const long long exc = sh.carry[x] + inc - term;
        if (here) wl.qprefix[x * row + i] = (int)min(exc, (long long)0x7fffffff);
        __syncthreads();
        // The last NQ threads hold each queue's chunk total.
        if (tid >= SCHED_THREADS - NQ) sh.carry[x] += inc;
        __syncthreads();
    }

    // ---- 3. totals and counters --------------------------------------------
    if (tid < NQ) {
        long long total = sh.carry[tid];
        if (total > 0x7fffffffLL) {
            flags |= 4;
            total = 0;  // refuse to run rather than wrap
        }
        const int pos = (full & 1) ? NQ - 1 - tid : tid;
        const int n = full + (pos < rem ? 1 : 0);
        wl.qprefix[tid * row + n] = (int)total;
        for (int set = 0; set < NSETS; ++set) wl.ctl[CTL_NEXT + CTL_LINE * (NQ * set + tid)] = 0;
        wl.ctl[CTL_TOTAL + tid] = (int)total;
    }
    if (flags) atomicOr(&sh.flags, flags);
    __syncthreads();
    if (tid == 0) {
        wl.ctl[CTL_FLAGS] = sh.flags;
        wl.ctl[CTL_MODE] = mode;
    }
}

}  // namespace

namespace {
__global__ void fill_ramp_kernel(int32_t* dst, int count, int step) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) dst[i] = i * step;
}
}  // namespace

namespace {
__global__ void clear_counters_kernel(int* ctl) {
    static_assert(NSETS * NQ <= 64, "one wave clears every counter");
    const int t = threadIdx.x;
    if (t < NSETS * NQ) ctl[CTL_NEXT + CTL_LINE * t] = 0;
}
}  // namespace

hipError_t launch_clear_counters(int* ctl, hipStream_t stream) {
    hipLaunchKernelGGL(clear_counters_kernel, dim3(1), dim3(64), 0, stream, ctl);
    return hipGetLastError();
}

hipError_t launch_fill_ramp(int32_t* dst, int count, int step, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_ramp_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, dst,
                       count, step);
    return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* offsets, int num_seqs, int heads, int q_tile_rows,
                           WorkList wl, hipStream_t stream, SortChoice choice, hipEvent_t start,
                           hipEvent_t stop) {
    int kind = RANK_COUNTING;
    if (choice == SortChoice::BITONIC) kind = RANK_BITONIC;
    if (choice == SortChoice::INPUT_ORDER) kind = RANK_INPUT;
    constexpr size_t counting_lds = sizeof(int) * (2 * (size_t)HIST_MAX + SORT_MAX);
    constexpr size_t bitonic_lds = sizeof(unsigned long long) * SORT_MAX;
    constexpr size_t max_lds = counting_lds > bitonic_lds ? counting_lds : bitonic_lds;
    size_t lds = 0;
    if (num_seqs <= SORT_MAX && kind != RANK_INPUT) {
        int P = 1;
        while (P < num_seqs) P <<= 1;
        const size_t need_bitonic = sizeof(unsigned long long) * (size_t)P;
        const size_t need_counting = sizeof(int) * (2 * (size_t)HIST_MAX + (size_t)num_seqs);
        // The device decides between counting and bitonic ranking, so provide both.
        lds = need_bitonic > need_counting ? need_bitonic : need_counting;
    }
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)schedule_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)max_lds);
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    if (start)
        hipExtLaunchKernelGGL(schedule_kernel, dim3(1), dim3(SCHED_THREADS), lds, stream, start,
                              stop, 0, offsets, num_seqs, heads, q_tile_rows, wl, kind);
    else
        hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(SCHED_THREADS), lds, stream, offsets,
                           num_seqs, heads, q_tile_rows, wl, kind);
    return hipGetLastError();
}

}  // namespace hstu
