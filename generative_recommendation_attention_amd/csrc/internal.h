// Internal declarations shared by the scheduler, the attention kernels and the
// C ABI layer.  Nothing here is part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

// Words at the start of the scratch area (int32).
enum : int {
    CTL_NEXT = 0,   // next work item to hand out (device atomic)
    CTL_TOTAL = 1,  // number of work items
    CTL_FLAGS = 2,  // bit 0: off[0] != 0, bit 1: a decreasing offset, bit 2: item count overflow
    CTL_MODE = 3,   // MODE_BANDS or MODE_SEQS
    CTL_WORDS = 16
};

// How work items are numbered.
//  MODE_BANDS: sequences are sorted by Q-tile count, longest first.  Items go in
//    order of decreasing Q-tile index j (the cost of an item is j + 1 key/value
//    tiles), so the heaviest items are handed out first.  Sorted rank m and the
//    next rank's count bound a "band" of levels in which exactly m + 1
//    sequences take part; prefix[m] is the first item of band m.
//  MODE_SEQS: sequences in input order, Q tiles of each from last to first;
//    prefix[i] is the first item of sequence i.  Used when there are more
//    sequences than the one-workgroup sort takes.
enum : int { MODE_BANDS = 0, MODE_SEQS = 1 };
constexpr int SORT_MAX = 16384;

struct WorkList {
    int* ctl;     // CTL_WORDS
    int* order;   // [num_seqs]      sequence id at each schedule rank
    int* ntile;   // [num_seqs + 1]  Q-tile count at each rank, then 0
    int* prefix;  // [num_seqs + 1]  first item of each band / sequence, then the total
};

inline size_t worklist_bytes(int num_seqs) {
    size_t n = (size_t)num_seqs;
    return sizeof(int) * (CTL_WORDS + n + 2 * (n + 1)) + 256;
}

inline WorkList worklist_carve(void* base, int num_seqs) {
    int* p = static_cast<int*>(base);
    WorkList wl;
    wl.ctl = p;
    wl.order = p + CTL_WORDS;
    wl.ntile = wl.order + num_seqs;
    wl.prefix = wl.ntile + num_seqs + 1;
    return wl;
}

hipError_t launch_schedule(const int32_t* offsets, int num_seqs, int heads, int q_tile_rows,
                           WorkList wl, hipStream_t stream);

enum class Dtype : int { BF16 = 0, FP16 = 1, FP32 = 2 };

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const int32_t* offsets;
    int num_seqs;
    int heads;
    int d;
    float alpha;
    float n;
};

// Rows of Q handled by one work item for this element type and head size.
int q_tile_rows(Dtype dt, int d);

// Enqueues the attention kernel (the work list must already be built on the
// same stream).  `grid` = 0 picks the resident-workgroup count of the device.
hipError_t launch_attention(const FwdParams& p, Dtype dt, WorkList wl, int grid,
                            hipStream_t stream);

}  // namespace hstu
