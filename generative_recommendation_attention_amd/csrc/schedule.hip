// Work-list build: one workgroup turns the jagged offsets into the numbering
// of work items that the attention kernel decodes (see schedule.h).
//
// Bands mode (num_seqs <= SORT_MAX): Q-tile counts are sorted in LDS (bitonic,
// descending, ties by sequence id) and the band prefix is a scan of
//   (ntile[m] - ntile[m+1]) * (m + 1) * heads.
// Sequences mode: identity order, prefix = scan of ntile[i] * heads.
// The kernel also resets the item counter, so a forward call needs no memset.
#include "internal.h"

namespace hstu {

namespace {

constexpr int SCHED_THREADS = 1024;

// Inclusive scan of one value per thread across the workgroup (64-bit).
__device__ long long block_inclusive_scan(long long x, long long* buf) {
    const int tid = threadIdx.x;
    buf[tid] = x;
    __syncthreads();
    for (int off = 1; off < SCHED_THREADS; off <<= 1) {
        long long y = (tid >= off) ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += y;
        __syncthreads();
    }
    long long r = buf[tid];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(SCHED_THREADS) void schedule_kernel(
        const int32_t* __restrict__ off, int num_seqs, int heads, int bq, WorkList wl,
        int mode) {
    extern __shared__ unsigned long long keys[];  // bands mode only
    __shared__ long long scan_buf[SCHED_THREADS];
    __shared__ int s_flags;
    const int tid = threadIdx.x;
    if (tid == 0) s_flags = 0;
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

    if (mode == MODE_BANDS) {
        int P = 1;
        while (P < num_seqs) P <<= 1;
        for (int i = tid; i < P; i += SCHED_THREADS) {
            unsigned long long key = 0;
            if (i < num_seqs)
                key = ((unsigned long long)(unsigned)tiles_of(i) << 32) |
                      (unsigned long long)(~(unsigned)i);
            keys[i] = key;
        }
        __syncthreads();
        // Bitonic sort, descending overall.
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
        for (int i = tid; i < num_seqs; i += SCHED_THREADS) {
            wl.order[i] = i;
            wl.ntile[i] = tiles_of(i);
        }
    }
    if (tid == 0) wl.ntile[num_seqs] = 0;

    // Exclusive scan of the per-rank item counts, in chunks of SCHED_THREADS.
    long long carry = 0;
    for (int base = 0; base < num_seqs; base += SCHED_THREADS) {
        const int m = base + tid;
        long long term = 0;
        if (m < num_seqs) {
            if (mode == MODE_BANDS) {
                const long long nm = (long long)(keys[m] >> 32);
                const long long nn = (m + 1 < num_seqs) ? (long long)(keys[m + 1] >> 32) : 0;
                term = (nm - nn) * (long long)(m + 1) * heads;
            } else {
                term = (long long)tiles_of(m) * heads;
            }
        }
        const long long inc = block_inclusive_scan(term, scan_buf);
        const long long exc = carry + inc - term;
        if (m < num_seqs) wl.prefix[m] = (int)min(exc, (long long)0x7fffffff);
        // The last thread's inclusive value is the chunk total.
        if (tid == SCHED_THREADS - 1) scan_buf[0] = inc;
        __syncthreads();
        carry += scan_buf[0];
        __syncthreads();
    }
    if (carry > 0x7fffffffLL) {
        flags |= 4;
        carry = 0;  // refuse to run rather than wrap
    }
    if (flags) atomicOr(&s_flags, flags);
    __syncthreads();
    if (tid == 0) {
        wl.prefix[num_seqs] = (int)carry;
        wl.ctl[CTL_NEXT] = 0;
        wl.ctl[CTL_TOTAL] = (int)carry;
        wl.ctl[CTL_FLAGS] = s_flags;
        wl.ctl[CTL_MODE] = mode;
    }
}

}  // namespace

hipError_t launch_schedule(const int32_t* offsets, int num_seqs, int heads, int q_tile_rows,
                           WorkList wl, hipStream_t stream) {
    const int mode = (num_seqs <= SORT_MAX) ? MODE_BANDS : MODE_SEQS;
    size_t lds = 0;
    if (mode == MODE_BANDS) {
        int P = 1;
        while (P < num_seqs) P <<= 1;
        lds = sizeof(unsigned long long) * (size_t)P;
    }
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t e = hipFuncSetAttribute((const void*)schedule_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(sizeof(unsigned long long) * SORT_MAX));
        if (e != hipSuccess) return e;
        attr_done = true;
    }
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(SCHED_THREADS), lds, stream, offsets,
                       num_seqs, heads, q_tile_rows, wl, mode);
    return hipGetLastError();
}

}  // namespace hstu
