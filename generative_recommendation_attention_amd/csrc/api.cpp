// C ABI of the HSTU forward (declared in include/hstu.h): argument checks on
// the host, the per-(device, stream) scratch area, event-based kernel timing,
// and the two launches (work list, attention) on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <list>
#include <map>
#include <memory>
#include <mutex>
#include <utility>
#include <vector>

#include "hstu.h"
#include "internal.h"

namespace {

thread_local int g_last_hip = 0;

hstu_status_t hip_fail(hipError_t e) {
    g_last_hip = (int)e;
    return HSTU_ERR_HIP;
}

// ---- scratch areas ----------------------------------------------------------

struct Scratch {
    void* ptr = nullptr;
    size_t bytes = 0;
    unsigned epoch = 0;   // counter sets consumed on this area; a call starts at set epoch % NSETS
    bool clean = false;   // sets epoch and epoch + 1 (mod NSETS) are known to be zero
    // Offsets i * len of the dense layout, written at ramp_at by an earlier
    // call on this area (ramp_count = 0: none).
    size_t ramp_at = 0;
    int ramp_count = 0;
    int64_t ramp_len = 0;
};

std::mutex g_scratch_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

// One call at a time per (device, stream): a call reads the area's counter-set
// rotation, may grow the area, launches, and then advances the rotation; two
// host threads interleaving those steps on one stream could share a counter
// set or see the area freed under them.  Held from before the scratch lookup
// to after the rotation is advanced (not for captured calls, which take an
// area of their own).
std::map<std::pair<int, hipStream_t>, std::unique_ptr<std::mutex>> g_call_mu;

std::unique_lock<std::mutex> stream_call_lock(int dev, hipStream_t stream, bool graph) {
    if (graph) return std::unique_lock<std::mutex>();
    std::mutex* m;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        auto& slot = g_call_mu[std::make_pair(dev, stream)];
        if (!slot) slot.reset(new std::mutex);
        m = slot.get();
    }
    return std::unique_lock<std::mutex>(*m);
}

// Returns a scratch area of at least `bytes` for (device, stream).  Growing an
// area first waits for the stream, so no kernel still reads the old one.
// A new area's contents are undefined (clean = false).
hstu_status_t scratch_for(int dev, hipStream_t stream, size_t bytes, Scratch** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    Scratch& s = g_scratch[std::make_pair(dev, stream)];
    if (s.bytes < bytes) {
        size_t want = bytes < 4096 ? 4096 : bytes;
        want = (want + 4095) & ~(size_t)4095;
        if (s.ptr) {
            hipError_t e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return hip_fail(e);
            (void)hipFree(s.ptr);
            s.ptr = nullptr;
            s.bytes = 0;
        }
        if (getenv("HSTU_FAIL_ALLOC") && atoi(getenv("HSTU_FAIL_ALLOC")) != 0)
            return HSTU_ERR_NO_MEMORY;
        void* p = nullptr;
        hipError_t e = hipMalloc(&p, want);
        if (e != hipSuccess) {
            g_last_hip = (int)e;
            return HSTU_ERR_NO_MEMORY;
        }
        s.ptr = p;
        s.bytes = want;
        s.epoch = 0;
        s.clean = false;
        s.ramp_count = 0;
    }
    *out = &s;
    return HSTU_OK;
}

// ---- calls captured into a graph ----------------------------------------------
//
// A graph keeps the addresses its kernels were captured with and replays them
// in any order relative to later eager calls, so a captured call shares no
// state with anything else: it gets a scratch area of its own, allocated
// during capture (the thread switches to relaxed capture mode for the
// allocation) and kept until the process ends, and its first captured kernel
// zeroes the area's counter sets, so that every replay starts from zero.
// Eager state (the per-stream area, its counter rotation and cached dense
// ramp) is left as it was.

std::list<Scratch> g_graph_areas;   // under g_scratch_mu; never freed

bool is_capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

hstu_status_t graph_scratch(size_t bytes, Scratch** out) {
    size_t want = bytes < 4096 ? 4096 : bytes;
    want = (want + 4095) & ~(size_t)4095;
    if (getenv("HSTU_FAIL_ALLOC") && atoi(getenv("HSTU_FAIL_ALLOC")) != 0)
        return HSTU_ERR_NO_MEMORY;
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    hipError_t e = hipThreadExchangeStreamCaptureMode(&mode);
    if (e != hipSuccess) return hip_fail(e);
    void* p = nullptr;
    e = hipMalloc(&p, want);
    (void)hipThreadExchangeStreamCaptureMode(&mode);   // the caller's mode again
    if (e != hipSuccess) {
        g_last_hip = (int)e;
        return HSTU_ERR_NO_MEMORY;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_graph_areas.emplace_back();
    Scratch& s = g_graph_areas.back();
    s.ptr = p;
    s.bytes = want;
    *out = &s;
    return HSTU_OK;
}

// The scratch area of one call and its first counter set (`sets` consecutive
// sets are used); *clean tells whether they are known to be zero.
hstu_status_t call_scratch(int dev, hipStream_t stream, bool graph, size_t bytes, Scratch** sc,
                           hstu::WorkList* wl, int num_seqs, int heads, bool* clean) {
    hstu_status_t st = graph ? graph_scratch(bytes, sc) : scratch_for(dev, stream, bytes, sc);
    if (st != HSTU_OK) return st;
    *wl = hstu::worklist_carve((*sc)->ptr, num_seqs, heads);
    if (graph) {
        const hipError_t e = hstu::launch_clear_counters(wl->ctl, stream);
        if (e != hipSuccess) return hip_fail(e);
        wl->set = 0;
        *clean = true;
        return HSTU_OK;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    wl->set = (int)((*sc)->epoch % hstu::NSETS);
    *clean = (*sc)->clean;
    (*sc)->clean = false;   // until this call's launches succeed
    return HSTU_OK;
}

// After a call's launches succeeded: `sets` counter sets consumed, and the
// launches cleared the next two (nothing to record for a captured call).
void call_done(Scratch* sc, bool graph, unsigned sets) {
    if (graph) return;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    sc->epoch += sets;
    sc->clean = true;
}

// A call whose work list reaches `bytes` into the area overwrites a dense
// offset ramp stored there.
void forget_ramp_under(Scratch* sc, size_t bytes) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (sc->ramp_count && bytes > sc->ramp_at) sc->ramp_count = 0;
}

// Offsets i * len (i = 0 .. num_seqs) of the dense layout at byte `at` of the
// area (which must hold them), written once per (area, num_seqs, len).
hstu_status_t dense_ramp(Scratch* sc, size_t at, int num_seqs, int64_t len, hipStream_t stream,
                         const int32_t** out) {
    int32_t* ramp = reinterpret_cast<int32_t*>(static_cast<char*>(sc->ptr) + at);
    bool have;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        have = sc->ramp_count == num_seqs && sc->ramp_len == len && sc->ramp_at == at;
    }
    if (!have) {
        hipError_t e = hstu::launch_fill_ramp(ramp, num_seqs + 1, (int)len, stream);
        if (e != hipSuccess) return hip_fail(e);
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        sc->ramp_count = num_seqs;
        sc->ramp_len = len;
        sc->ramp_at = at;
    }
    *out = ramp;
    return HSTU_OK;
}

// ---- device checks ----------------------------------------------------------

std::mutex g_dev_mu;
std::map<int, bool> g_dev_ok;

hstu_status_t check_device(int* dev_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    *dev_out = dev;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    auto it = g_dev_ok.find(dev);
    if (it == g_dev_ok.end()) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        it = g_dev_ok.emplace(dev, ok).first;
    }
    return it->second ? HSTU_OK : HSTU_ERR_UNSUPPORTED;
}

// ---- kernel timing ----------------------------------------------------------

// Start and stop events of the work-list kernel (e[0], e[1], recorded only when
// it runs) and of the attention kernel (e[2], e[3]).  They are attached to the
// kernel dispatches themselves, so timing adds no packets to the stream.
struct TimedCall {
    hipEvent_t e[4];
    bool sched = false;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<TimedCall> g_prof_pending;
std::vector<TimedCall> g_prof_free;
hstu_kernel_times_t g_prof_total = {0, 0.0, 0.0, 0, 0.0, 0.0, 0.0};
std::vector<float> g_prof_attn;   // per-call attention-kernel times since the last reset
// Per-device clock record of timed forward calls (CLK_SLOTS workgroups,
// CLK_WORDS words each), the id the last timed call wrote and its device.
std::map<int, unsigned long long*> g_clk_buf;
unsigned g_clk_next = 0;
int g_clk_last_dev = -1;
unsigned g_clk_last_id = 0;

// The clock record for a timed call on `dev` (allocated on first use), or
// null if that fails; *id receives the call's id.
unsigned long long* clock_slot(int dev, unsigned* id) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    unsigned long long*& b = g_clk_buf[dev];
    if (!b) {
        void* ptr = nullptr;
        if (hipMalloc(&ptr, sizeof(unsigned long long) * hstu::CLK_WORDS * hstu::CLK_SLOTS) !=
            hipSuccess)
            return nullptr;
        b = static_cast<unsigned long long*>(ptr);
    }
    *id = ++g_clk_next;
    g_clk_last_dev = dev;
    g_clk_last_id = *id;
    return b;
}
constexpr size_t PROF_RING = 4096;

bool prof_take(TimedCall* tc) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    if (!g_prof_on) return false;
    if (g_prof_pending.size() >= PROF_RING) {
        g_prof_total.dropped++;
        return false;
    }
    if (!g_prof_free.empty()) {
        *tc = g_prof_free.back();
        g_prof_free.pop_back();
        return true;
    }
    for (int i = 0; i < 4; ++i) {
        if (hipEventCreate(&tc->e[i]) != hipSuccess) {
            for (int j = 0; j < i; ++j) (void)hipEventDestroy(tc->e[j]);
            g_prof_total.dropped++;
            return false;
        }
    }
    return true;
}

void prof_commit(const TimedCall& tc) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_pending.push_back(tc);
}

// ---- argument checks --------------------------------------------------------

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hstu_status_t check_args(const void* q, const void* k, const void* v, const int32_t* off,
                         int32_t num_seqs, int32_t heads, int32_t d, float alpha, float n,
                         const void* out, int dtype) {
    if (dtype != HSTU_BF16 && dtype != HSTU_FP16 && dtype != HSTU_FP32) return HSTU_ERR_UNSUPPORTED;
    if (num_seqs < 0 || heads < 1) return HSTU_ERR_INVALID_ARG;
    if ((long long)num_seqs * heads > 0x7fffffffLL) return HSTU_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return HSTU_ERR_UNSUPPORTED;
    if (!std::isfinite(alpha) || !std::isfinite(n) || n == 0.0f) return HSTU_ERR_INVALID_ARG;
    if (num_seqs == 0) return HSTU_OK;
    if (!q || !k || !v || !off || !out) return HSTU_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return HSTU_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(off) & 3u) != 0) return HSTU_ERR_INVALID_ARG;
    if (out == q || out == k || out == v) return HSTU_ERR_INVALID_ARG;
    return HSTU_OK;
}

bool validate_env() {
    const char* s = getenv("HSTU_VALIDATE");
    return s && atoi(s) != 0;
}

// HSTU_SCHED_SORT=bitonic|input forces one ranking path of the scheduler.
hstu::SortChoice sort_choice_env() {
    const char* s = getenv("HSTU_SCHED_SORT");
    if (!s) return hstu::SortChoice::AUTO;
    if (std::strcmp(s, "bitonic") == 0) return hstu::SortChoice::BITONIC;
    if (std::strcmp(s, "input") == 0) return hstu::SortChoice::INPUT_ORDER;
    return hstu::SortChoice::AUTO;
}

// Extra inputs of the masked forms: candidate counts (target-aware mask), or
// a cached history (K, V and their offsets); all null for the causal mask.
struct MaskInputs {
    const int32_t* num_targets = nullptr;
    const void* k_cache = nullptr;
    const void* v_cache = nullptr;
    const int32_t* hist_offsets = nullptr;
    // Dense (B, heads, S, D) layout: num_seqs = B, dense_len = S, no offsets.
    bool dense = false;
    int64_t dense_len = 0;
    // Relative attention bias.
    const int32_t* timestamps = nullptr;
    const int32_t* hist_timestamps = nullptr;   // with a cached history
    const float* pos_bias = nullptr;
    const float* time_bias = nullptr;
    int num_pos = 0;
    int num_time = 0;
};

// One forward call.
// fixed_area: the caller's device area of fixed_bytes for the work list (the
// allocation-free entry point), instead of the library's per-stream scratch.
// Such a call keeps no host-side state: it zeroes the queue counters itself.
hstu_status_t attn_fwd_call(const void* q, const void* k, const void* v,
                            const int32_t* seq_offsets, const MaskInputs& mi, int32_t num_seqs,
                            int32_t heads, int32_t d, float alpha, float n, void* out,
                            hipStream_t stream, int dtype, void* fixed_area = nullptr,
                            size_t fixed_bytes = 0) {
    // (the dense entry point checks its own arguments and passes no offsets)
    hstu_status_t st = mi.dense ? HSTU_OK
                                : check_args(q, k, v, seq_offsets, num_seqs, heads, d, alpha, n,
                                             out, dtype);
    if (st != HSTU_OK || num_seqs == 0) return st;
    int dev = 0;
    st = check_device(&dev);
    if (st != HSTU_OK) return st;

    const hstu::Dtype dt = static_cast<hstu::Dtype>(dtype);
    const bool graph = is_capturing(stream);
    const bool fixed = fixed_area != nullptr;
    const std::unique_lock<std::mutex> call_lock = stream_call_lock(dev, stream, graph || fixed);
    Scratch* sc = nullptr;
    const size_t wl_bytes = (hstu::worklist_bytes(num_seqs, heads) + 255) & ~(size_t)255;
    const size_t ramp_bytes = mi.dense ? sizeof(int32_t) * ((size_t)num_seqs + 1) : 0;
    hstu::WorkList wl;
    bool clean;
    // Small batches build their queue tables inside the attention kernel.  The
    // work-list kernel still runs when this call's counter set is not known to
    // be zero (a new scratch area, or a failed launch before; it zeroes both
    // sets) and when a test forces one of its ranking paths.
    const hstu::SortChoice sort = sort_choice_env();
    const bool fusable = sort == hstu::SortChoice::AUTO && num_seqs <= hstu::FUSE_SEQS &&
                         (long long)num_seqs * heads <= hstu::FUSE_PAIRS;
    if (fixed) {
        if (mi.dense) return HSTU_ERR_INVALID_ARG;
        if (wl_bytes > fixed_bytes) return HSTU_ERR_SCRATCH_LIMIT;
        wl = hstu::worklist_carve(fixed_area, num_seqs, heads);
        wl.set = 0;
        // The one-kernel form needs counter set 0 at zero: a one-wave kernel
        // clears every set first (the work-list kernel of the two-kernel form
        // clears them itself).
        clean = fusable;
        if (fusable) {
            const hipError_t e = hstu::launch_clear_counters(wl.ctl, stream);
            if (e != hipSuccess) return hip_fail(e);
        }
    } else {
        st = call_scratch(dev, stream, graph, wl_bytes + ramp_bytes, &sc, &wl, num_seqs, heads,
                          &clean);
        if (st != HSTU_OK) return st;
        forget_ramp_under(sc, wl_bytes);
        if (mi.dense) {
            st = dense_ramp(sc, wl_bytes, num_seqs, mi.dense_len, stream, &seq_offsets);
            if (st != HSTU_OK) return st;
        }
    }
    wl.fused = clean && fusable;

    hstu::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.offsets = seq_offsets;
    p.num_targets = mi.num_targets;
    p.k_cache = mi.k_cache;
    p.v_cache = mi.v_cache;
    p.hist_offsets = mi.hist_offsets;
    p.dense = mi.dense;
    p.dense_len = mi.dense_len;
    p.timestamps = mi.timestamps;
    p.hist_timestamps = mi.hist_timestamps;
    p.pos_bias = mi.pos_bias;
    p.time_bias = mi.time_bias;
    p.num_pos = mi.num_pos;
    p.num_time = mi.num_time;
    p.num_seqs = num_seqs;
    p.heads = heads;
    p.d = d;
    p.alpha = alpha;
    p.n = n;

    TimedCall tc;
    // (the allocation-free form is never timed: timing creates events and a
    // clock buffer)
    const bool timed = !graph && !fixed && prof_take(&tc);
    if (timed) p.clk = clock_slot(dev, &p.clk_id);
    tc.sched = false;
    hipError_t e;
    if (!wl.fused) {
        const int rows =
                hstu::q_tile_rows(dt, d, mi.hist_offsets != nullptr || mi.timestamps != nullptr);
        e = hstu::launch_schedule(seq_offsets, num_seqs, heads, rows, wl, stream, sort,
                                  timed ? tc.e[0] : nullptr, timed ? tc.e[1] : nullptr);
        if (e != hipSuccess) return hip_fail(e);
        tc.sched = timed;
    }
    e = hstu::launch_attention(p, dt, wl, 0, stream, timed ? tc.e[2] : nullptr,
                               timed ? tc.e[3] : nullptr);
    if (e != hipSuccess) return hip_fail(e);
    if (!fixed) call_done(sc, graph, 1);   // one counter set used, the next two cleared
    if (timed) prof_commit(tc);
    if (!graph && validate_env()) {
        int ctl[hstu::CTL_WORDS];
        e = hipMemcpyAsync(ctl, wl.ctl, sizeof ctl, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e);
        if (ctl[hstu::CTL_FLAGS] != 0) return HSTU_ERR_BAD_OFFSETS;
    }
    return HSTU_OK;
}

// One backward call: the dK/dV kernel, then the dQ kernel, on one work list
// of BWD_TILE_ROWS-row items (a counter set per kernel).
// dense_len > 0: the dense (B, heads, S, d) layout with S = dense_len, no offsets.
// The relative-attention-bias inputs and table-gradient outputs of a
// backward call (null: no bias).
struct RabGrads {
    const int32_t* timestamps;
    const float* pos_bias;
    const float* time_bias;
    int num_pos;
    int num_time;
    float* d_pos_bias;
    float* d_time_bias;
};

hstu_status_t attn_bwd_call(const void* q, const void* k, const void* v, const void* dout,
                            const int32_t* seq_offsets, const int32_t* num_targets,
                            int32_t num_seqs, int32_t heads, int32_t d, float alpha, float n,
                            void* dq, void* dk, void* dv, hipStream_t stream, int dtype,
                            int64_t dense_len = 0, const RabGrads* rab = nullptr) {
    // (a dense call has no offsets yet: q stands in for the pointer check)
    const int32_t* off_check = dense_len > 0 ? reinterpret_cast<const int32_t*>(q) : seq_offsets;
    hstu_status_t st = check_args(q, k, v, off_check, num_seqs, heads, d, alpha, n, dq, dtype);
    if (st != HSTU_OK) return st;
    if (num_seqs == 0) return HSTU_OK;
    if (!dout || !dk || !dv) return HSTU_ERR_INVALID_ARG;
    if (!aligned16(dout) || !aligned16(dk) || !aligned16(dv)) return HSTU_ERR_INVALID_ARG;
    const void* ins[4] = {q, k, v, dout};
    const void* outs[3] = {dq, dk, dv};
    for (const void* o : outs)
        for (const void* i : ins)
            if (o == i) return HSTU_ERR_INVALID_ARG;
    if (dq == dk || dq == dv || dk == dv) return HSTU_ERR_INVALID_ARG;
    int dev = 0;
    st = check_device(&dev);
    if (st != HSTU_OK) return st;

    const hstu::Dtype dt = static_cast<hstu::Dtype>(dtype);
    const bool graph = is_capturing(stream);
    const std::unique_lock<std::mutex> call_lock = stream_call_lock(dev, stream, graph);
    Scratch* sc = nullptr;
    const size_t wl_bytes = (hstu::worklist_bytes(num_seqs, heads) + 255) & ~(size_t)255;
    const size_t ramp_bytes = dense_len > 0 ? sizeof(int32_t) * ((size_t)num_seqs + 1) : 0;
    const size_t part_bytes =
            rab ? sizeof(float) * (size_t)hstu::RAB_PARTS * hstu::rab_partial_stride(rab->num_pos)
                : 0;
    hstu::WorkList wl;
    bool clean;
    st = call_scratch(dev, stream, graph, wl_bytes + ramp_bytes + part_bytes, &sc, &wl, num_seqs,
                      heads, &clean);
    if (st != HSTU_OK) return st;
    // (the bias partials follow the work list and overwrite what was there)
    forget_ramp_under(sc, wl_bytes + part_bytes);
    if (dense_len > 0) {
        st = dense_ramp(sc, wl_bytes, num_seqs, dense_len, stream, &seq_offsets);
        if (st != HSTU_OK) return st;
    }
    const hstu::SortChoice sort = sort_choice_env();
    wl.fused = clean && sort == hstu::SortChoice::AUTO && num_seqs <= hstu::FUSE_SEQS &&
               (long long)num_seqs * heads <= hstu::FUSE_PAIRS;

    hstu::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.offsets = seq_offsets;
    p.num_targets = num_targets;
    p.dense = dense_len > 0;
    p.dense_len = dense_len;
    if (rab) {
        p.timestamps = rab->timestamps;
        p.pos_bias = rab->pos_bias;
        p.time_bias = rab->time_bias;
        p.num_pos = rab->num_pos;
        p.num_time = rab->num_time;
        p.d_pos_bias = rab->d_pos_bias;
        p.d_time_bias = rab->d_time_bias;
        p.rab_partials = reinterpret_cast<float*>(static_cast<char*>(sc->ptr) + wl_bytes);
    }
    p.num_seqs = num_seqs;
    p.heads = heads;
    p.d = d;
    p.alpha = alpha;
    p.n = n;

    TimedCall tc;
    const bool timed = !graph && prof_take(&tc);
    tc.sched = false;
    hipError_t e;
    if (!wl.fused) {
        e = hstu::launch_schedule(seq_offsets, num_seqs, heads, hstu::BWD_TILE_ROWS, wl, stream,
                                  sort, timed ? tc.e[0] : nullptr, timed ? tc.e[1] : nullptr);
        if (e != hipSuccess) return hip_fail(e);
        tc.sched = timed;
    }
    e = hstu::launch_backward(p, dt, wl, stream, timed ? tc.e[2] : nullptr,
                              timed ? tc.e[3] : nullptr);
    if (e != hipSuccess) return hip_fail(e);
    call_done(sc, graph, 2);   // two launches, two counter sets; the next two cleared
    if (timed) prof_commit(tc);
    return HSTU_OK;
}

}  // namespace

namespace hstu {

hstu_status_t attn_fwd_fixed_area(const void* q, const void* k, const void* v,
                                  const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                  int32_t d, float alpha, float n, void* out, hipStream_t stream,
                                  int dtype, void* area, size_t area_bytes) {
    if (!area || area_bytes == 0) return HSTU_ERR_INVALID_ARG;
    return attn_fwd_call(q, k, v, seq_offsets, MaskInputs{}, num_seqs, heads, d, alpha, n, out,
                         stream, dtype, area, area_bytes);
}

hstu_status_t hip_error_status(hipError_t e) { return hip_fail(e); }

}  // namespace hstu

extern "C" {

hstu_status_t hstu_attn_fwd(const void* q, const void* k, const void* v,
                            const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                            int32_t d, float alpha, float n, void* out, hipStream_t stream,
                            hstu_dtype_t dtype) {
    return attn_fwd_call(q, k, v, seq_offsets, MaskInputs{}, num_seqs, heads, d, alpha, n, out,
                         stream, dtype);
}

hstu_status_t hstu_attn_fwd_targets(const void* q, const void* k, const void* v,
                                    const int32_t* seq_offsets, const int32_t* num_targets,
                                    int32_t num_seqs, int32_t heads, int32_t d, float alpha,
                                    float n, void* out, hipStream_t stream, hstu_dtype_t dtype) {
    if (num_seqs > 0 && (!num_targets || (reinterpret_cast<uintptr_t>(num_targets) & 3u) != 0))
        return HSTU_ERR_INVALID_ARG;
    MaskInputs mi;
    mi.num_targets = num_targets;
    return attn_fwd_call(q, k, v, seq_offsets, mi, num_seqs, heads, d, alpha, n, out, stream,
                         dtype);
}

// The bias inputs of a forward call, checked (num_seqs > 0: non-null and
// 4-byte aligned tables and timestamps).
static hstu_status_t rab_inputs(const int32_t* timestamps, const float* pos_bias,
                                int32_t num_pos, const float* time_bias, int32_t num_time,
                                int32_t num_seqs, float alpha, MaskInputs* mi) {
    if (num_pos < 1 || num_pos > (1 << 28) || num_time < 1 || num_time > 32)
        return HSTU_ERR_INVALID_ARG;
    // The kernels carry the bias in units of the raw score (rab / alpha).
    if (!(alpha != 0.0f) || !std::isfinite((float)(1.0 / (double)alpha)))
        return HSTU_ERR_INVALID_ARG;
    if (num_seqs > 0) {
        const uintptr_t bad = reinterpret_cast<uintptr_t>(timestamps) |
                              reinterpret_cast<uintptr_t>(pos_bias) |
                              reinterpret_cast<uintptr_t>(time_bias);
        if (!timestamps || !pos_bias || !time_bias || (bad & 3u) != 0) return HSTU_ERR_INVALID_ARG;
    }
    mi->timestamps = timestamps;
    mi->pos_bias = pos_bias;
    mi->time_bias = time_bias;
    mi->num_pos = num_pos;
    mi->num_time = num_time;
    return HSTU_OK;
}

hstu_status_t hstu_attn_fwd_rab(const void* q, const void* k, const void* v,
                                const int32_t* seq_offsets, const int32_t* timestamps,
                                const float* pos_bias, int32_t num_pos, const float* time_bias,
                                int32_t num_time, int32_t num_seqs, int32_t heads, int32_t d,
                                float alpha, float n, void* out, hipStream_t stream,
                                hstu_dtype_t dtype) {
    MaskInputs mi;
    const hstu_status_t st =
            rab_inputs(timestamps, pos_bias, num_pos, time_bias, num_time, num_seqs, alpha, &mi);
    if (st != HSTU_OK) return st;
    return attn_fwd_call(q, k, v, seq_offsets, mi, num_seqs, heads, d, alpha, n, out, stream,
                         dtype);
}

hstu_status_t hstu_attn_fwd_rab_targets(const void* q, const void* k, const void* v,
                                        const int32_t* seq_offsets, const int32_t* num_targets,
                                        const int32_t* timestamps, const float* pos_bias,
                                        int32_t num_pos, const float* time_bias,
                                        int32_t num_time, int32_t num_seqs, int32_t heads,
                                        int32_t d, float alpha, float n, void* out,
                                        hipStream_t stream, hstu_dtype_t dtype) {
    if (num_seqs > 0 && (!num_targets || (reinterpret_cast<uintptr_t>(num_targets) & 3u) != 0))
        return HSTU_ERR_INVALID_ARG;
    MaskInputs mi;
    const hstu_status_t st =
            rab_inputs(timestamps, pos_bias, num_pos, time_bias, num_time, num_seqs, alpha, &mi);
    if (st != HSTU_OK) return st;
    mi.num_targets = num_targets;
    return attn_fwd_call(q, k, v, seq_offsets, mi, num_seqs, heads, d, alpha, n, out, stream,
                         dtype);
}

hstu_status_t hstu_attn_fwd_dense(const void* q, const void* k, const void* v, int32_t batch,
                                  int32_t heads, int32_t seq_len, int32_t d, float alpha, float n,
                                  void* out, hipStream_t stream, hstu_dtype_t dtype) {
    if (dtype != HSTU_BF16 && dtype != HSTU_FP16 && dtype != HSTU_FP32) return HSTU_ERR_UNSUPPORTED;
    if (batch < 0 || heads < 1 || seq_len < 0) return HSTU_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return HSTU_ERR_UNSUPPORTED;
    if ((long long)batch * seq_len > 0x7fffffffLL || (long long)batch * heads > 0x7fffffffLL)
        return HSTU_ERR_UNSUPPORTED;
    if (!std::isfinite(alpha) || !std::isfinite(n) || n == 0.0f) return HSTU_ERR_INVALID_ARG;
    if (batch == 0 || seq_len == 0) return HSTU_OK;
    if (!q || !k || !v || !out) return HSTU_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return HSTU_ERR_INVALID_ARG;
    if (out == q || out == k || out == v) return HSTU_ERR_INVALID_ARG;
    MaskInputs mi;
    mi.dense = true;
    mi.dense_len = seq_len;
    return attn_fwd_call(q, k, v, nullptr, mi, batch, heads, d, alpha, n, out, stream, dtype);
}

hstu_status_t hstu_layer_in_proj(const void* x, const void* w1, const float* b1,
                                 int64_t num_tokens, int32_t d_model, int32_t heads, int32_t d,
                                 void* u, void* v, void* q, void* k, hipStream_t stream,
                                 hstu_dtype_t dtype) {
    if (dtype == HSTU_FP32) return HSTU_ERR_UNSUPPORTED;
    if (dtype != HSTU_BF16 && dtype != HSTU_FP16) return HSTU_ERR_UNSUPPORTED;
    if (num_tokens < 0 || heads < 1 || d < 1) return HSTU_ERR_INVALID_ARG;
    const long long hd = (long long)heads * d;
    if ((d_model != 128 && d_model != 256 && d_model != 512) ||
        (hd != 128 && hd != 256 && hd != 512))
        return HSTU_ERR_UNSUPPORTED;
    if (num_tokens > (1LL << 40)) return HSTU_ERR_UNSUPPORTED;
    if (num_tokens == 0) return HSTU_OK;
    const void* ptrs[8] = {x, w1, b1, u, v, q, k, nullptr};
    for (int i = 0; i < 7; ++i)
        if (!ptrs[i] || !aligned16(ptrs[i])) return HSTU_ERR_INVALID_ARG;
    const void* outs[4] = {u, v, q, k};
    for (int i = 0; i < 4; ++i) {
        if (outs[i] == x || outs[i] == w1 || outs[i] == b1) return HSTU_ERR_INVALID_ARG;
        for (int j = 0; j < i; ++j)
            if (outs[i] == outs[j]) return HSTU_ERR_INVALID_ARG;
    }
    int dev = 0;
    hstu_status_t st = check_device(&dev);
    if (st != HSTU_OK) return st;
    hstu::LayerParams p;
    p.x = x;
    p.w1 = w1;
    p.b1 = b1;
    p.uvqk[0] = u;
    p.uvqk[1] = v;
    p.uvqk[2] = q;
    p.uvqk[3] = k;
    p.T = num_tokens;
    p.d_model = d_model;
    p.heads_d = (int)hd;
    hipError_t e = hstu::launch_layer_in(p, static_cast<hstu::Dtype>(dtype), stream);
    return e == hipSuccess ? HSTU_OK : hip_fail(e);
}

hstu_status_t hstu_layer_out_proj(const void* attn, const void* u, const void* x,
                                  const float* gamma, const float* beta, float eps,
                                  const void* w2, const float* b2, int64_t num_tokens,
                                  int32_t d_model, int32_t heads, int32_t d, void* y,
                                  hipStream_t stream, hstu_dtype_t dtype) {
    if (dtype == HSTU_FP32) return HSTU_ERR_UNSUPPORTED;
    if (dtype != HSTU_BF16 && dtype != HSTU_FP16) return HSTU_ERR_UNSUPPORTED;
    if (num_tokens < 0 || heads < 1 || d < 1) return HSTU_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f) return HSTU_ERR_INVALID_ARG;
    const long long hd = (long long)heads * d;
    if ((d_model != 128 && d_model != 256 && d_model != 512) ||
        (hd != 128 && hd != 256 && hd != 512))
        return HSTU_ERR_UNSUPPORTED;
    if (num_tokens > (1LL << 40)) return HSTU_ERR_UNSUPPORTED;
    if (num_tokens == 0) return HSTU_OK;
    const void* ins[7] = {attn, u, x, gamma, beta, w2, b2};
    for (const void* pin : ins)
        if (!pin || !aligned16(pin)) return HSTU_ERR_INVALID_ARG;
    if (!y || !aligned16(y)) return HSTU_ERR_INVALID_ARG;
    for (const void* pin : ins)
        if (y == pin) return HSTU_ERR_INVALID_ARG;
    int dev = 0;
    hstu_status_t st = check_device(&dev);
    if (st != HSTU_OK) return st;
    hstu::LayerParams p;
    p.attn = attn;
    p.u = u;
    p.x = x;
    p.gamma = gamma;
    p.beta = beta;
    p.eps = eps;
    p.w2 = w2;
    p.b2 = b2;
    p.y = y;
    p.T = num_tokens;
    p.d_model = d_model;
    p.heads_d = (int)hd;
    hipError_t e = hstu::launch_layer_out(p, static_cast<hstu::Dtype>(dtype), stream);
    return e == hipSuccess ? HSTU_OK : hip_fail(e);
}

hstu_status_t hstu_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                            const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                            int32_t d, float alpha, float n, void* dq, void* dk, void* dv,
                            hipStream_t stream, hstu_dtype_t dtype) {
    return attn_bwd_call(q, k, v, dout, seq_offsets, nullptr, num_seqs, heads, d, alpha, n, dq,
                         dk, dv, stream, dtype);
}

hstu_status_t hstu_attn_bwd_targets(const void* q, const void* k, const void* v,
                                    const void* dout, const int32_t* seq_offsets,
                                    const int32_t* num_targets, int32_t num_seqs, int32_t heads,
                                    int32_t d, float alpha, float n, void* dq, void* dk,
                                    void* dv, hipStream_t stream, hstu_dtype_t dtype) {
    if (num_seqs > 0 && (!num_targets || (reinterpret_cast<uintptr_t>(num_targets) & 3u) != 0))
        return HSTU_ERR_INVALID_ARG;
    return attn_bwd_call(q, k, v, dout, seq_offsets, num_targets, num_seqs, heads, d, alpha, n,
                         dq, dk, dv, stream, dtype);
}

// (shared checks of the two bias backward entry points)
static hstu_status_t attn_bwd_rab_call(const void* q, const void* k, const void* v,
                                       const void* dout, const int32_t* seq_offsets,
                                       const int32_t* num_targets, const int32_t* timestamps,
                                       const float* pos_bias, int32_t num_pos,
                                       const float* time_bias, int32_t num_time,
                                       int32_t num_seqs, int32_t heads, int32_t d, float alpha,
                                       float n, void* dq, void* dk, void* dv, float* d_pos_bias,
                                       float* d_time_bias, hipStream_t stream,
                                       hstu_dtype_t dtype) {
    if (num_pos < 1 || num_pos > (1 << 18) || num_time < 1 || num_time > 32)
        return HSTU_ERR_INVALID_ARG;
    if (!(alpha != 0.0f) || !std::isfinite((float)(1.0 / (double)alpha)))
        return HSTU_ERR_INVALID_ARG;
    if (num_seqs > 0) {
        const uintptr_t bad = reinterpret_cast<uintptr_t>(timestamps) |
                              reinterpret_cast<uintptr_t>(pos_bias) |
                              reinterpret_cast<uintptr_t>(time_bias) |
                              reinterpret_cast<uintptr_t>(d_pos_bias) |
                              reinterpret_cast<uintptr_t>(d_time_bias);
        if (!timestamps || !pos_bias || !time_bias || !d_pos_bias || !d_time_bias ||
            (bad & 3u) != 0)
            return HSTU_ERR_INVALID_ARG;
    }
    const RabGrads rab{timestamps, pos_bias, time_bias, num_pos, num_time, d_pos_bias,
                       d_time_bias};
    return attn_bwd_call(q, k, v, dout, seq_offsets, num_targets, num_seqs, heads, d, alpha, n,
                         dq, dk, dv, stream, dtype, 0, &rab);
}

hstu_status_t hstu_attn_bwd_rab(const void* q, const void* k, const void* v, const void* dout,
                                const int32_t* seq_offsets, const int32_t* timestamps,
                                const float* pos_bias, int32_t num_pos, const float* time_bias,
                                int32_t num_time, int32_t num_seqs, int32_t heads, int32_t d,
                                float alpha, float n, void* dq, void* dk, void* dv,
                                float* d_pos_bias, float* d_time_bias, hipStream_t stream,
                                hstu_dtype_t dtype) {
    return attn_bwd_rab_call(q, k, v, dout, seq_offsets, nullptr, timestamps, pos_bias, num_pos,
                             time_bias, num_time, num_seqs, heads, d, alpha, n, dq, dk, dv,
                             d_pos_bias, d_time_bias, stream, dtype);
}

hstu_status_t hstu_attn_bwd_rab_targets(const void* q, const void* k, const void* v,
                                        const void* dout, const int32_t* seq_offsets,
                                        const int32_t* num_targets, const int32_t* timestamps,
                                        const float* pos_bias, int32_t num_pos,
                                        const float* time_bias, int32_t num_time,
                                        int32_t num_seqs, int32_t heads, int32_t d, float alpha,
                                        float n, void* dq, void* dk, void* dv, float* d_pos_bias,
                                        float* d_time_bias, hipStream_t stream,
                                        hstu_dtype_t dtype) {
    if (num_seqs > 0 && (!num_targets || (reinterpret_cast<uintptr_t>(num_targets) & 3u) != 0))
        return HSTU_ERR_INVALID_ARG;
    return attn_bwd_rab_call(q, k, v, dout, seq_offsets, num_targets, timestamps, pos_bias,
                             num_pos, time_bias, num_time, num_seqs, heads, d, alpha, n, dq, dk,
                             dv, d_pos_bias, d_time_bias, stream, dtype);
}

hstu_status_t hstu_attn_bwd_dense(const void* q, const void* k, const void* v, const void* dout,
                                  int32_t batch, int32_t heads, int32_t seq_len, int32_t d,
                                  float alpha, float n, void* dq, void* dk, void* dv,
                                  hipStream_t stream, hstu_dtype_t dtype) {
    if (dtype != HSTU_BF16 && dtype != HSTU_FP16 && dtype != HSTU_FP32) return HSTU_ERR_UNSUPPORTED;
    if (batch < 0 || heads < 1 || seq_len < 0) return HSTU_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return HSTU_ERR_UNSUPPORTED;
    if ((long long)batch * seq_len > 0x7fffffffLL || (long long)batch * heads > 0x7fffffffLL)
        return HSTU_ERR_UNSUPPORTED;
    if (!std::isfinite(alpha) || !std::isfinite(n) || n == 0.0f) return HSTU_ERR_INVALID_ARG;
    if (batch == 0 || seq_len == 0) return HSTU_OK;
    return attn_bwd_call(q, k, v, dout, nullptr, nullptr, batch, heads, d, alpha, n, dq, dk, dv,
                         stream, dtype, seq_len);
}

// The cache inputs of a cached-history call, checked (num_seqs > 0).
static hstu_status_t cache_inputs(const void* k_cache, const void* v_cache,
                                  const int32_t* hist_offsets, const void* out, int32_t num_seqs,
                                  MaskInputs* mi) {
    if (num_seqs > 0) {
        // Both caches null: no request has a history (T_hist = 0).
        if (!hist_offsets || (!k_cache) != (!v_cache)) return HSTU_ERR_INVALID_ARG;
        if (!aligned16(k_cache) || !aligned16(v_cache)) return HSTU_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(hist_offsets) & 3u) != 0) return HSTU_ERR_INVALID_ARG;
        if (out == k_cache || out == v_cache) return HSTU_ERR_INVALID_ARG;
    }
    mi->k_cache = k_cache;
    mi->v_cache = v_cache;
    mi->hist_offsets = hist_offsets;
    return HSTU_OK;
}

hstu_status_t hstu_attn_fwd_cached(const void* q, const void* k, const void* v,
                                   const int32_t* cand_offsets, const void* k_cache,
                                   const void* v_cache, const int32_t* hist_offsets,
                                   int32_t num_seqs, int32_t heads, int32_t d, float alpha,
                                   float n, void* out, hipStream_t stream, hstu_dtype_t dtype) {
    MaskInputs mi;
    const hstu_status_t st = cache_inputs(k_cache, v_cache, hist_offsets, out, num_seqs, &mi);
    if (st != HSTU_OK) return st;
    return attn_fwd_call(q, k, v, cand_offsets, mi, num_seqs, heads, d, alpha, n, out, stream,
                         dtype);
}

hstu_status_t hstu_attn_fwd_rab_cached(const void* q, const void* k, const void* v,
                                       const int32_t* cand_offsets, const void* k_cache,
                                       const void* v_cache, const int32_t* hist_offsets,
                                       const int32_t* timestamps,
                                       const int32_t* hist_timestamps, const float* pos_bias,
                                       int32_t num_pos, const float* time_bias,
                                       int32_t num_time, int32_t num_seqs, int32_t heads,
                                       int32_t d, float alpha, float n, void* out,
                                       hipStream_t stream, hstu_dtype_t dtype) {
    MaskInputs mi;
    hstu_status_t st = cache_inputs(k_cache, v_cache, hist_offsets, out, num_seqs, &mi);
    if (st != HSTU_OK) return st;
    st = rab_inputs(timestamps, pos_bias, num_pos, time_bias, num_time, num_seqs, alpha, &mi);
    if (st != HSTU_OK) return st;
    // (a history needs its timestamps; with no cache there is no history)
    if (num_seqs > 0 && k_cache &&
        (!hist_timestamps || (reinterpret_cast<uintptr_t>(hist_timestamps) & 3u) != 0))
        return HSTU_ERR_INVALID_ARG;
    mi.hist_timestamps = k_cache ? hist_timestamps : nullptr;
    return attn_fwd_call(q, k, v, cand_offsets, mi, num_seqs, heads, d, alpha, n, out, stream,
                         dtype);
}

hstu_status_t hstu_attn_fwd_bf16(const void* q, const void* k, const void* v,
                                 const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                 int32_t d, float alpha, float n, void* out, hipStream_t stream) {
    return hstu_attn_fwd(q, k, v, seq_offsets, num_seqs, heads, d, alpha, n, out, stream,
                         HSTU_BF16);
}

hstu_status_t hstu_attn_fwd_fp16(const void* q, const void* k, const void* v,
                                 const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                 int32_t d, float alpha, float n, void* out, hipStream_t stream) {
    return hstu_attn_fwd(q, k, v, seq_offsets, num_seqs, heads, d, alpha, n, out, stream,
                         HSTU_FP16);
}

hstu_status_t hstu_attn_fwd_fp32(const void* q, const void* k, const void* v,
                                 const int32_t* seq_offsets, int32_t num_seqs, int32_t heads,
                                 int32_t d, float alpha, float n, void* out, hipStream_t stream) {
    return hstu_attn_fwd(q, k, v, seq_offsets, num_seqs, heads, d, alpha, n, out, stream,
                         HSTU_FP32);
}

hstu_status_t hstu_validate_offsets(const int32_t* seq_offsets, int32_t num_seqs,
                                    int64_t* total, hipStream_t stream) {
    if (num_seqs < 0) return HSTU_ERR_INVALID_ARG;
    if (num_seqs > 0 && !seq_offsets) return HSTU_ERR_INVALID_ARG;
    if (num_seqs == 0) {
        if (total) *total = 0;
        return HSTU_OK;
    }
    std::vector<int32_t> h((size_t)num_seqs + 1);
    hipError_t e = hipMemcpyAsync(h.data(), seq_offsets, sizeof(int32_t) * h.size(),
                                  hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e);
    if (total) *total = h[num_seqs];
    if (h[0] != 0) return HSTU_ERR_BAD_OFFSETS;
    for (int32_t i = 0; i < num_seqs; ++i)
        if (h[i + 1] < h[i]) return HSTU_ERR_BAD_OFFSETS;
    return HSTU_OK;
}

const char* hstu_status_string(hstu_status_t status) {
    switch (status) {
    case HSTU_OK: return "ok";
    case HSTU_ERR_INVALID_ARG: return "invalid argument";
    case HSTU_ERR_UNSUPPORTED: return "unsupported head size, element type or device";
    case HSTU_ERR_HIP: return "HIP runtime error";
    case HSTU_ERR_NO_MEMORY: return "scratch allocation failed";
    case HSTU_ERR_BAD_OFFSETS: return "malformed sequence offsets";
    case HSTU_ERR_SCRATCH_LIMIT: return "work list larger than the fixed scratch area";
    }
    return "unknown status";
}

int hstu_last_hip_error(void) { return g_last_hip; }

void hstu_release_workspace(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (auto it = g_scratch.begin(); it != g_scratch.end();) {
        if (it->first.first == dev) {
            if (it->second.ptr) (void)hipFree(it->second.ptr);
            it = g_scratch.erase(it);
        } else {
            ++it;
        }
    }
}

hstu_status_t hstu_profile_enable(int on) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_on = on != 0;
    return HSTU_OK;
}

hstu_status_t hstu_profile_read(hstu_kernel_times_t* out, int reset) {
    if (!out) return HSTU_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_prof_mu);
    for (const TimedCall& tc : g_prof_pending) {
        hipError_t e = hipEventSynchronize(tc.e[3]);
        if (e != hipSuccess) return hip_fail(e);
        float a = 0.f, b = 0.f;
        e = tc.sched ? hipEventElapsedTime(&a, tc.e[0], tc.e[1]) : hipSuccess;
        if (e == hipSuccess) e = hipEventElapsedTime(&b, tc.e[2], tc.e[3]);
        if (e != hipSuccess) return hip_fail(e);
        g_prof_total.calls++;
        g_prof_total.sched_ms += a;
        g_prof_total.attn_ms += b;
        g_prof_attn.push_back(b);
        g_prof_free.push_back(tc);
    }
    g_prof_pending.clear();
    if (!g_prof_attn.empty()) {
        std::vector<float> t(g_prof_attn);
        std::sort(t.begin(), t.end());
        const size_t m = t.size();
        g_prof_total.attn_min_ms = t[0];
        g_prof_total.attn_median_ms = m % 2 ? t[m / 2] : 0.5 * ((double)t[m / 2 - 1] + t[m / 2]);
    }
    // The clock of the last timed forward call: per workgroup, the shader
    // clock counter's advance over the 100 MHz counter's, averaged.
    g_prof_total.clock_mhz = 0.0;
    if (g_clk_last_dev >= 0 && g_clk_last_id != 0) {
        std::vector<unsigned long long> h((size_t)hstu::CLK_WORDS * hstu::CLK_SLOTS);
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess) e = hipSetDevice(g_clk_last_dev);
        if (e == hipSuccess)
            e = hipMemcpy(h.data(), g_clk_buf[g_clk_last_dev], h.size() * sizeof(h[0]),
                          hipMemcpyDeviceToHost);
        (void)hipSetDevice(cur);
        if (e != hipSuccess) return hip_fail(e);
        double sum = 0.0;
        int cnt = 0;
        for (int w = 0; w < hstu::CLK_SLOTS; ++w) {
            const unsigned long long* r = &h[(size_t)hstu::CLK_WORDS * w];
            if (r[4] != g_clk_last_id || r[3] <= r[1]) continue;
            sum += 100.0 * (double)(r[2] - r[0]) / (double)(r[3] - r[1]);
            ++cnt;
        }
        if (cnt) g_prof_total.clock_mhz = sum / cnt;
    }
    *out = g_prof_total;
    if (reset) {
        g_prof_total = hstu_kernel_times_t{0, 0.0, 0.0, 0, 0.0, 0.0, 0.0};
        g_prof_attn.clear();
        g_clk_last_id = 0;
    }
    return HSTU_OK;
}

}  // extern "C"
