// Internal declarations shared by the scheduler, the attention kernels and the
// C ABI layer.  Nothing here is part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hstu.h"

namespace hstu {

// The forward (causal mask, jagged layout) with its work list in `area`
// (area_bytes long) instead of the library's per-stream scratch: used by the
// allocation-free entry point.  Allocates nothing and keeps no host state.
hstu_status_t attn_fwd_fixed_area(const void* q, const void* k, const void* v,
                                  const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                  int32_t d, float alpha, float n, void* out, hipStream_t stream,
                                  int dtype, void* area, size_t area_bytes);
// Records e as the calling thread's last HIP error; returns HSTU_ERR_HIP.
hstu_status_t hip_error_status(hipError_t e);

// Work items are (sequence, head, Q tile) triples, split over NQ queues (one
// per XCD of an MI355X; a workgroup starts with the queue of the XCD it runs
// on, so the items sharing one sequence's keys and values run under one L2).
constexpr int NQ = 8;
constexpr int CTL_LINE = 32;  // ints per queue counter: one 128-byte line each
// Queue counter sets.  A call takes one (forward) or two (backward: one per
// pass) consecutive sets, and clears the two after them, so whichever call
// comes next finds its sets at zero.
constexpr int NSETS = 4;

// Words at the start of the scratch area (int32).
enum : int {
    CTL_NEXT = 0,                 // NEXT + CTL_LINE*(NQ*set + x): next item of queue x for
                                  // counter set `set` (0 .. NSETS-1; device atomic)
    CTL_TOTAL = NSETS * NQ * CTL_LINE,  // TOTAL + x: items in queue x
    CTL_FLAGS = CTL_TOTAL + NQ,   // bit 0: off[0] != 0, bit 1: a decreasing offset,
                                  // bit 2: item count overflow
    CTL_MODE = CTL_FLAGS + 1,     // QUEUE_BANDS or QUEUE_PAIRS
    CTL_WORDS = CTL_TOTAL + 2 * NQ
};
static_assert(CTL_MODE < CTL_WORDS, "control block layout");

// Small batches skip the work-list kernel: every workgroup of the attention
// kernel ranks the sequences and builds the queue tables itself, in LDS, at
// its start (the tables are a few KB; building them costs less than a second
// kernel launch).  Up to FUSE_SEQS sequences and FUSE_PAIRS (sequence, head)
// pairs.  Either way the queue counters are zero when a launch starts: calls
// on one work list rotate through NSETS counter sets, and each launch clears
// the sets the next call will use (the work-list kernel clears all).
constexpr int FUSE_SEQS = 256;
constexpr int FUSE_PAIRS = 2048;
constexpr int FUSE_QLEN = FUSE_PAIRS / NQ;

// QUEUE_BANDS: ranks sorted, items level by level (below).  QUEUE_PAIRS: items
// pair by pair, each pair's Q tiles from last to first; qprefix then holds
// each pair's first item.  Pairs are used in input order (more sequences than
// the sort takes), and for sorted ranks when no sequence has more than
// PAIRS_MAX_TILES Q tiles: a batch of short sequences is balanced either way,
// and with a pair's tiles next to each other in the queue they run at about
// the same time on one XCD, so the later tile's key/value reads hit the L2
// (measured on 4096 sequences of U[1, 256] tokens, d 128: reads 1.33x -> 1.00x
// of the algorithmic bytes, 0.332 -> 0.310 ms).  Level order keeps the long
// sequences' largest tiles first, which their balance needs.
enum : int { QUEUE_BANDS = 0, QUEUE_PAIRS = 1 };
constexpr int PAIRS_MAX_TILES = 2;

// The scheduler ranks sequences by Q-tile count, largest first (or keeps input
// order above SORT_MAX sequences).  Pairs p = rank * heads + head are dealt to
// the queues in snake order: round i = p / NQ goes to queues 0..NQ-1 when i is
// even and NQ-1..0 when odd, so heavy pairs spread evenly.  Inside a queue,
// whose pairs are then in non-increasing tile count, items go level by level
// from the last Q tile down: the level-j items of every pair with more than j
// tiles, pair by pair.  "Band" b of a queue holds the levels in which exactly
// its first b + 1 pairs take part; qprefix holds each band's first item.
constexpr int SORT_MAX = 16384;

// Pair dealt to position i of queue x.
__host__ __device__ inline int queue_pair(int i, int x) {
    return i * NQ + ((i & 1) ? NQ - 1 - x : x);
}

struct WorkList {
    int* ctl;      // CTL_WORDS
    int* order;    // [num_seqs]      sequence id at each rank
    int* ntile;    // [num_seqs]      Q-tile count at each rank
    int* qprefix;  // [NQ * (qlen + 1)] first item of each band of a queue, then the total
    int qlen;      // max pairs per queue = ceil(num_seqs * heads / NQ)
    int fused;     // 1: the attention kernel builds the tables in LDS (FUSE_* limits)
    int set;       // first counter set of this call (0 .. NSETS-1)
};

// The tables item decoding reads: the work list in global memory, or the
// copy a workgroup built in its LDS (generic pointers to either).
struct Tables {
    const int* order;
    const int* ntile;
    const int* qprefix;
    const int* totals;   // [NQ]
    int qlen;
    int mode;            // QUEUE_BANDS or QUEUE_PAIRS
};

// LDS copy of the tables for a fused launch.
struct LocalTables {
    int order[FUSE_SEQS];
    int ntile[FUSE_SEQS];
    int qprefix[NQ * (FUSE_QLEN + 1)];
    int totals[NQ];
    int flags;
};

inline int queue_len(int num_seqs, int heads) {
    const long long pairs = (long long)num_seqs * heads;
    return (int)((pairs + NQ - 1) / NQ);
}

inline size_t worklist_bytes(int num_seqs, int heads) {
    const size_t qlen = (size_t)queue_len(num_seqs, heads);
    return sizeof(int) * (CTL_WORDS + 2 * (size_t)num_seqs + NQ * (qlen + 1)) + 256;
}

inline WorkList worklist_carve(void* base, int num_seqs, int heads) {
    int* p = static_cast<int*>(base);
    WorkList wl;
    wl.ctl = p;
    wl.order = p + CTL_WORDS;
    wl.ntile = wl.order + num_seqs;
    wl.qprefix = wl.ntile + num_seqs;
    wl.qlen = queue_len(num_seqs, heads);
    wl.fused = 0;
    wl.set = 0;
    return wl;
}

// How the scheduler ranks sequences.  AUTO: counting sort on tile counts
// (bitonic sort if a count is too large for its histogram; input order above
// SORT_MAX sequences).  The other two force one path, for tests.
enum class SortChoice : int { AUTO = 0, BITONIC = 1, INPUT_ORDER = 2 };

// `start` / `stop`, when not null, are recorded by the kernel dispatch itself
// (timing without extra stream packets).
hipError_t launch_schedule(const int32_t* offsets, int num_seqs, int heads, int q_tile_rows,
                           WorkList wl, hipStream_t stream, SortChoice choice,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

enum class Dtype : int { BF16 = 0, FP16 = 1, FP32 = 2 };

// Writes dst[i] = i * step for i < count (offsets of equal-length sequences).
hipError_t launch_fill_ramp(int32_t* dst, int count, int step, hipStream_t stream);
// Zeroes every counter set of the work list whose control block is ctl (one
// small kernel): the first kernel of a call captured into a graph, so that
// each replay starts from zero counters without a memset node.
hipError_t launch_clear_counters(int* ctl, hipStream_t stream);

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const int32_t* offsets;
    const int32_t* num_targets;   // candidates per sequence, or null (plain causal)
    // Cached-history form (offsets, q, k, v, out are then the candidates'):
    const void* k_cache;          // history K, V (T_hist, heads, d), or null
    const void* v_cache;
    const int32_t* hist_offsets;  // int32[num_seqs + 1], or null (not the cached form)
    // Dense (B, heads, S, D) layout: offsets are then i * S, S = dense_len.
    bool dense = false;
    int64_t dense_len = 0;
    // Relative attention bias (jagged layout only): token timestamps (T),
    // position table [num_pos], time table [num_time <= 32]; with a cached
    // history also the history's timestamps (T_hist).
    const int32_t* timestamps = nullptr;
    const int32_t* hist_timestamps = nullptr;
    const float* pos_bias = nullptr;
    const float* time_bias = nullptr;
    int num_pos = 0;
    int num_time = 0;
    int num_seqs;
    int heads;
    int d;
    float alpha;
    float n;
    // Timed calls only: workgroup w of the attention kernel writes
    // clk[CLK_WORDS w + 0..4] = shader-clock counter and 100 MHz counter at
    // its start, the same at its end, then clk_id (w < CLK_SLOTS), or null.
    unsigned long long* clk = nullptr;
    unsigned clk_id = 0;
};
constexpr int CLK_WORDS = 8;
constexpr int CLK_SLOTS = 4096;

// Rows of Q handled by one work item for this element type and head size;
// single_block: the cached-history and relative-attention-bias forms, whose
// waves hold one 32-row block each.
int q_tile_rows(Dtype dt, int d, bool single_block = false);

// Compute units of the current device.
int device_cus();

// Workgroups of `fn` (with `threads` threads) that fit on the device at once.
template <typename KernelFn>
int resident_grid(KernelFn fn, int threads) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    return per_cu * device_cus();
}

// The layer's surroundings (bf16 / fp16): input projection with SiLU and
// split, layer norm times U with output projection and residual.
struct LayerParams {
    // layer_in
    const void* x = nullptr;       // (T, d_model)
    const void* w1 = nullptr;      // (4 heads d, d_model)
    const float* b1 = nullptr;     // [4 heads d]
    void* uvqk[4] = {nullptr, nullptr, nullptr, nullptr};   // each (T, heads, d)
    // layer_out
    const void* attn = nullptr;    // (T, heads, d)
    const void* u = nullptr;       // (T, heads, d)
    const float* gamma = nullptr;  // [heads d]
    const float* beta = nullptr;   // [heads d]
    const void* w2 = nullptr;      // (d_model, heads d)
    const float* b2 = nullptr;     // [d_model]
    void* y = nullptr;             // (T, d_model)
    float eps = 0.0f;
    int64_t T = 0;
    int d_model = 0;
    int heads_d = 0;
};

hipError_t launch_layer_in(const LayerParams& p, Dtype dt, hipStream_t stream);
hipError_t launch_layer_out(const LayerParams& p, Dtype dt, hipStream_t stream);

// Backward: gradients of the forward with respect to q, k and v for an
// upstream gradient dout (bf16 / fp16 only).  Work items are 128-row tiles of
// each (sequence, head): the work list must be built with BWD_TILE_ROWS.
constexpr int BWD_TILE_ROWS = 128;

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    const int32_t* offsets;
    const int32_t* num_targets;   // candidates per sequence, or null (plain causal)
    bool dense = false;           // dense (B, heads, S, D) layout, S = dense_len
    int64_t dense_len = 0;
    // Relative attention bias (bf16 / fp16, jagged causal): the forward's
    // inputs, the tables' gradients (fp32, overwritten) and the partials
    // buffer (RAB_PARTS * rab_partial_stride(num_pos) floats of scratch).
    const int32_t* timestamps = nullptr;
    const float* pos_bias = nullptr;
    const float* time_bias = nullptr;
    int num_pos = 0;
    int num_time = 0;
    float* d_pos_bias = nullptr;
    float* d_time_bias = nullptr;
    float* rab_partials = nullptr;
    int num_seqs;
    int heads;
    int d;
    float alpha;
    float n;
};

// Table-gradient partials of the bias backward: workgroup w of the dQ kernel
// adds to partial w % RAB_PARTS (global atomics), so a few workgroups share
// one; a last kernel sums the partials.
constexpr int RAB_PARTS = 64;
inline int rab_partial_stride(int num_pos) { return (num_pos + 32 + 63) / 64 * 64; }

// Enqueues the dK/dV kernel (counter set wl.set) and then the dQ kernel (the
// next set); each clears one of the two sets after those.  `start` / `stop`,
// when given, are recorded on the first and second dispatch.
hipError_t launch_backward(const BwdParams& p, Dtype dt, WorkList wl, hipStream_t stream,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Enqueues the attention kernel (the work list must already be built on the
// same stream).  `grid` = 0 picks the resident-workgroup count of the device.
hipError_t launch_attention(const FwdParams& p, Dtype dt, WorkList wl, int grid,
                            hipStream_t stream, hipEvent_t start = nullptr,
                            hipEvent_t stop = nullptr);

}  // namespace hstu
