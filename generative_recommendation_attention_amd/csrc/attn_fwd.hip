// HSTU jagged causal attention forward on gfx950 matrix cores.
//
//   out[r] = (1/n) * sum_{c <= r} silu(alpha <q_r, k_c>) v_c      (per sequence, head)
//
// Ascend HSTU blog ("都是生成式推荐，为什么昇腾这么快？"): §1 gives the formula
// and its five unfused steps; §2.1-§2.2 fuse them so the (s x s) score matrix
// stays on chip, block by block, and the (block x d) result is accumulated;
// §3.2 builds the causal mask inside the operator (full / lower-triangular /
// skipped block pairs); §4.2 takes jagged values + offsets.  On gfx950 the
// score tile lives in MFMA accumulators, the pointwise pass runs on them in
// registers, and the weights feed the second product without leaving the
// register file.
//
// Persistent workgroups pull items (sequence, head, Q tile) from the work list
// built by schedule.hip.  Per item, each wave owns 32 query rows and walks the
// key/value tiles 0..(last tile that reaches its rows), staged through LDS and
// double buffered: while tile c is consumed, tile c+1 is in flight from HBM.
//
// Transposed products.  With v_mfma_f32_32x32x16_{bf16,f16} a lane's C/D
// registers hold one column and 16 rows of a 32x32 block:
//   column = lane % 32,  row = 8*(r/4) + 4*(lane/32) + r%4   (r = register 0..15).
// Computing S^T = K Q^T (keys down, queries across) therefore leaves each lane
// with one query and 16 keys, which is the k-slice the second product
// O^T = V^T P^T needs in its B operand.  The keys a lane holds for k-step t are
// {16t + 8*(e/4) + 4*(lane/32) + e%4 : e = 0..7}; V^T is stored in LDS with
// bits 2 and 3 of the key index swapped inside each group of 16, so a lane's
// eight matching V values are one contiguous 16-byte read.
//
// Scaling.  With m = -alpha*log2(e)*s, silu(alpha*s) = -(m / log2(e)) *
// 1/(1 + 2^m).  The kernel forms p = m * rcp(1 + exp2(m)) (one multiply, two
// transcendental instructions, one add, one multiply per score) and applies
// -ln(2)/n to the accumulated output once, in the epilogue.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "schedule.h"

namespace hstu {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct KernelArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    const int32_t* offsets;
    WorkList wl;
    int num_seqs;
    int heads;
    float score_scale;  // -alpha * log2(e)
    float out_scale;    // -ln(2) / n
};

template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mfma<_Float16> {
    typedef f16x8 v8;
    typedef f16x4 v4;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// Position in LDS of key `kv` inside its group of 16: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int kv) {
    return (kv & ~12) | ((kv & 4) << 1) | ((kv & 8) >> 1);
}

// -log2(e) * silu(alpha*s), given m = -alpha*log2(e)*s.
__device__ __forceinline__ float silu_scaled(float m) {
    const float t = __builtin_amdgcn_exp2f(m);
    return m * __builtin_amdgcn_rcpf(1.0f + t);
}

// ---------------------------------------------------------------------------
// bf16 / fp16: one wave = 32 query rows; NW waves per workgroup.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int BK>
struct Tile16 {
    static constexpr int BQ = NW * 32;              // query rows per item
    static constexpr int THREADS = NW * 64;
    static constexpr int KSTR = D + 8;              // K row stride in LDS (elements)
    static constexpr int VSTR = BK + 8;             // V^T row stride in LDS (elements)
    static constexpr int K_ELEMS = BK * KSTR;
    static constexpr int V_ELEMS = D * VSTR;
    static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
    static constexpr int K_CHUNKS = BK * D / 8 / THREADS;   // 16-byte K loads per thread
    static constexpr int V_UNITS = BK * D / 16 / THREADS;   // (2 rows x 8 cols) V units per thread
    static_assert(K_CHUNKS * THREADS * 8 == BK * D, "K tile must split evenly");
    static_assert(V_UNITS * THREADS * 16 == BK * D, "V tile must split evenly");
    static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
};

template <typename T, int D, int NW, int BK>
__global__ __launch_bounds__(NW * 64) void attn_fwd_mfma16(KernelArgs a) {
    using Cfg = Tile16<T, D, NW, BK>;
    using M = Mfma<T>;
    using v8 = typename M::v8;
    using v4 = typename M::v4;
    constexpr int BQ = Cfg::BQ;
    constexpr int KSTR = Cfg::KSTR;
    constexpr int VSTR = Cfg::VSTR;

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * Cfg::BUF_ELEMS];
    __shared__ int s_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = (int64_t)H * D;  // elements between consecutive tokens
    const int total = a.wl.ctl[CTL_TOTAL];
    const int mode = a.wl.ctl[CTL_MODE];

    for (;;) {
        if (tid == 0) s_item = atomicAdd(a.wl.ctl + CTL_NEXT, 1);
        __syncthreads();
        const int w = s_item;
        if (w >= total) break;
        const Item it = decode_item(a.wl, mode, a.num_seqs, H, w);
        const int start = a.offsets[it.seq];
        const int s = a.offsets[it.seq + 1] - start;
        const int q0 = it.qtile * BQ;
        const int kv_end = min(s, q0 + BQ);
        const int n_tiles = (kv_end + BK - 1) / BK;
        const int wr0 = q0 + wv * 32;  // this wave's first query row (local)
        const bool wave_live = wr0 < s;
        const int my_row = wr0 + l32;
        const int64_t head_off = (int64_t)it.head * D;
        const int64_t seq_base = (int64_t)start * row_stride + head_off;

        // Q^T operand: query my_row, head-dim slice [16*ks + 8*g, +8).
        v8 qop[D / 16];
        {
            const uint4* qp = reinterpret_cast<const uint4*>(a.q + seq_base +
                                                            (int64_t)my_row * row_stride);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                uint4 x = make_uint4(0, 0, 0, 0);
                if (my_row < s) x = qp[ks * 2 + g];
                qop[ks] = __builtin_bit_cast(v8, x);
            }
        }
        f32x16 o[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};

        // Staging registers for one K/V tile.
        uint4 kreg[Cfg::K_CHUNKS];
        uint4 vreg[Cfg::V_UNITS][2];

        auto load_tile = [&](int c) {
            const int k0 = c * BK;
#pragma unroll
            for (int i = 0; i < Cfg::K_CHUNKS; ++i) {
                const int id = tid + i * Cfg::THREADS;
                const int r = id / (D / 8), c8 = id % (D / 8);
                uint4 x = make_uint4(0, 0, 0, 0);
                if (k0 + r < s)
                    x = *reinterpret_cast<const uint4*>(a.k + seq_base +
                                                        (int64_t)(k0 + r) * row_stride + c8 * 8);
                kreg[i] = x;
            }
#pragma unroll
            for (int i = 0; i < Cfg::V_UNITS; ++i) {
                const int id = tid + i * Cfg::THREADS;
                const int rp = id / (D / 8), c8 = id % (D / 8);
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int r = 2 * rp + h2;
                    uint4 x = make_uint4(0, 0, 0, 0);
                    if (k0 + r < s)
                        x = *reinterpret_cast<const uint4*>(
                                a.v + seq_base + (int64_t)(k0 + r) * row_stride + c8 * 8);
                    vreg[i][h2] = x;
                }
            }
        };
        auto store_tile = [&](int buf) {
            uint16_t* kl = lds + buf * Cfg::BUF_ELEMS;
            uint16_t* vl = kl + Cfg::K_ELEMS;
#pragma unroll
            for (int i = 0; i < Cfg::K_CHUNKS; ++i) {
                const int id = tid + i * Cfg::THREADS;
                const int r = id / (D / 8), c8 = id % (D / 8);
                *reinterpret_cast<uint4*>(kl + r * KSTR + c8 * 8) = kreg[i];
            }
#pragma unroll
            for (int i = 0; i < Cfg::V_UNITS; ++i) {
                const int id = tid + i * Cfg::THREADS;
                const int rp = id / (D / 8), c8 = id % (D / 8);
                const int pos = vt_pos(2 * rp);
                const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&vreg[i][0]);
                const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&vreg[i][1]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo = (x0[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                    const uint32_t hi = (x1[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                    *reinterpret_cast<uint32_t*>(vl + (c8 * 8 + e) * VSTR + pos) = lo | (hi << 16);
                }
            }
        };

        load_tile(0);
        store_tile(0);
        __syncthreads();

        for (int c = 0; c < n_tiles; ++c) {
            const bool more = c + 1 < n_tiles;
            if (more) load_tile(c + 1);
            const int k0 = c * BK;
            const bool skip = !wave_live || k0 > wr0 + 31;
            if (!skip) {
                const uint16_t* kl = lds + (c & 1) * Cfg::BUF_ELEMS;
                const uint16_t* vl = kl + Cfg::K_ELEMS;
                const bool partial = k0 + BK - 1 > wr0;
                // S^T = K Q^T, one 32-key block at a time.
                f32x16 st[BK / 32];
#pragma unroll
                for (int kb = 0; kb < BK / 32; ++kb) {
                    st[kb] = (f32x16){};
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks) {
                        const v8 ka = *reinterpret_cast<const v8*>(
                                kl + (kb * 32 + l32) * KSTR + ks * 16 + g * 8);
                        st[kb] = M::mma(ka, qop[ks], st[kb]);
                    }
                }
                // Pointwise pass and the second product, per 16-key step.
#pragma unroll
                for (int kb = 0; kb < BK / 32; ++kb) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        f32x8 pf;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            float p = silu_scaled(st[kb][8 * t + e] * a.score_scale);
                            if (partial) {
                                const int kv = k0 + kb * 32 + 16 * t + 8 * (e >> 2) + 4 * g + (e & 3);
                                p = (kv <= my_row) ? p : 0.0f;
                            }
                            pf[e] = p;
                        }
                        const v8 pb = __builtin_convertvector(pf, v8);
#pragma unroll
                        for (int db = 0; db < D / 32; ++db) {
                            const v8 va = *reinterpret_cast<const v8*>(
                                    vl + (db * 32 + l32) * VSTR + (kb * 2 + t) * 16 + g * 8);
                            o[db] = M::mma(va, pb, o[db]);
                        }
                    }
                }
            }
            if (more) store_tile((c + 1) & 1);
            __syncthreads();
        }

        // Epilogue: lane holds query my_row, head-dim rows 32*db + 8*i + 4*g + (0..3).
        if (my_row < s) {
            uint16_t* op = a.out + seq_base + (int64_t)my_row * row_stride;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 x;
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = o[db][4 * i + j] * a.out_scale;
                    const v4 y = __builtin_convertvector(x, v4);
                    *reinterpret_cast<v4*>(op + db * 32 + 8 * i + 4 * g) = y;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32: v_mfma_f32_32x32x2_f32.  A lane's k-slice is one element, and S^T's
// register r is already the B operand of k-step r of the second product (its
// key is 8*(r/4) + 4*(lane/32) + r%4), so no reordering is needed at all.
// ---------------------------------------------------------------------------
template <int D, int NW, int BK>
struct TileF32 {
    static constexpr int BQ = NW * 32;
    static constexpr int THREADS = NW * 64;
    static constexpr int KSTR = D + 2;   // floats
    static constexpr int VSTR = D + 8;   // floats
    static constexpr int CHUNKS = BK * D / 4 / THREADS;  // 16-byte loads per thread per tensor
    static_assert(CHUNKS * THREADS * 4 == BK * D, "tile must split evenly");
};

struct KernelArgsF32 {
    const float* q;
    const float* k;
    const float* v;
    float* out;
    const int32_t* offsets;
    WorkList wl;
    int num_seqs;
    int heads;
    float score_scale;
    float out_scale;
};

template <int D, int NW, int BK>
__global__ __launch_bounds__(NW * 64) void attn_fwd_mfma_f32(KernelArgsF32 a) {
    using Cfg = TileF32<D, NW, BK>;
    constexpr int BQ = Cfg::BQ;
    __shared__ __attribute__((aligned(16))) float kl[BK * Cfg::KSTR];
    __shared__ __attribute__((aligned(16))) float vl[BK * Cfg::VSTR];
    __shared__ int s_item;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = (int64_t)H * D;
    const int total = a.wl.ctl[CTL_TOTAL];
    const int mode = a.wl.ctl[CTL_MODE];

    for (;;) {
        if (tid == 0) s_item = atomicAdd(a.wl.ctl + CTL_NEXT, 1);
        __syncthreads();
        const int w = s_item;
        if (w >= total) break;
        const Item it = decode_item(a.wl, mode, a.num_seqs, H, w);
        const int start = a.offsets[it.seq];
        const int s = a.offsets[it.seq + 1] - start;
        const int q0 = it.qtile * BQ;
        const int kv_end = min(s, q0 + BQ);
        const int n_tiles = (kv_end + BK - 1) / BK;
        const int wr0 = q0 + wv * 32;
        const bool wave_live = wr0 < s;
        const int my_row = wr0 + l32;
        const int64_t seq_base = (int64_t)start * row_stride + (int64_t)it.head * D;

        float qf[D / 2];
        {
            const float* qp = a.q + seq_base + (int64_t)my_row * row_stride;
#pragma unroll
            for (int ks = 0; ks < D / 2; ++ks) qf[ks] = (my_row < s) ? qp[2 * ks + g] : 0.0f;
        }
        f32x16 o[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};

        for (int c = 0; c < n_tiles; ++c) {
            const int k0 = c * BK;
#pragma unroll
            for (int i = 0; i < Cfg::CHUNKS; ++i) {
                const int id = tid + i * Cfg::THREADS;
                const int r = id / (D / 4), c4 = id % (D / 4);
                float4 xk = make_float4(0.f, 0.f, 0.f, 0.f), xv = xk;
                if (k0 + r < s) {
                    const int64_t off = seq_base + (int64_t)(k0 + r) * row_stride + c4 * 4;
                    xk = *reinterpret_cast<const float4*>(a.k + off);
                    xv = *reinterpret_cast<const float4*>(a.v + off);
                }
                float* kd = kl + r * Cfg::KSTR + c4 * 4;
                kd[0] = xk.x; kd[1] = xk.y; kd[2] = xk.z; kd[3] = xk.w;
                *reinterpret_cast<float4*>(vl + r * Cfg::VSTR + c4 * 4) = xv;
            }
            __syncthreads();
            const bool skip = !wave_live || k0 > wr0 + 31;
            if (!skip) {
                const bool partial = k0 + BK - 1 > wr0;
#pragma unroll
                for (int kb = 0; kb < BK / 32; ++kb) {
                    f32x16 st = (f32x16){};
#pragma unroll
                    for (int ks = 0; ks < D / 2; ++ks)
                        st = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                kl[(kb * 32 + l32) * Cfg::KSTR + 2 * ks + g], qf[ks], st, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kvl = kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                        float p = silu_scaled(st[r] * a.score_scale);
                        if (partial) p = (k0 + kvl <= my_row) ? p : 0.0f;
#pragma unroll
                        for (int db = 0; db < D / 32; ++db)
                            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                    vl[kvl * Cfg::VSTR + db * 32 + l32], p, o[db], 0, 0, 0);
                    }
                }
            }
            __syncthreads();
        }

        if (my_row < s) {
            float* op = a.out + seq_base + (int64_t)my_row * row_stride;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float4 x;
                    x.x = o[db][4 * i + 0] * a.out_scale;
                    x.y = o[db][4 * i + 1] * a.out_scale;
                    x.z = o[db][4 * i + 2] * a.out_scale;
                    x.w = o[db][4 * i + 3] * a.out_scale;
                    *reinterpret_cast<float4*>(op + db * 32 + 8 * i + 4 * g) = x;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Launch configuration per (element type, head size).
// ---------------------------------------------------------------------------
constexpr int NW16 = 4;
constexpr int BK16 = 64;
constexpr int NWF = 4;
constexpr int BKF = 32;

struct DeviceInfo {
    int cus = 0;
};

int device_cus() {
    static thread_local int cached_dev = -1;
    static thread_local int cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

template <typename KernelFn>
int resident_grid(KernelFn fn, int threads) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    return per_cu * device_cus();
}

template <typename T, int D>
hipError_t launch16(const FwdParams& p, WorkList wl, int grid, hipStream_t stream) {
    KernelArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.out = static_cast<uint16_t*>(p.out);
    a.offsets = p.offsets;
    a.wl = wl;
    a.num_seqs = p.num_seqs;
    a.heads = p.heads;
    a.score_scale = -p.alpha * LOG2E;
    a.out_scale = -LN2 / p.n;
    auto fn = attn_fwd_mfma16<T, D, NW16, BK16>;
    if (grid <= 0) {
        static int cached = 0;
        if (!cached) cached = resident_grid(fn, NW16 * 64);
        grid = cached;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NW16 * 64), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const FwdParams& p, WorkList wl, int grid, hipStream_t stream) {
    KernelArgsF32 a;
    a.q = static_cast<const float*>(p.q);
    a.k = static_cast<const float*>(p.k);
    a.v = static_cast<const float*>(p.v);
    a.out = static_cast<float*>(p.out);
    a.offsets = p.offsets;
    a.wl = wl;
    a.num_seqs = p.num_seqs;
    a.heads = p.heads;
    a.score_scale = -p.alpha * LOG2E;
    a.out_scale = -LN2 / p.n;
    auto fn = attn_fwd_mfma_f32<D, NWF, BKF>;
    if (grid <= 0) {
        static int cached = 0;
        if (!cached) cached = resident_grid(fn, NWF * 64);
        grid = cached;
    }
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NWF * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

int q_tile_rows(Dtype dt, int d) {
    (void)d;
    return dt == Dtype::FP32 ? TileF32<64, NWF, BKF>::BQ : Tile16<__bf16, 64, NW16, BK16>::BQ;
}

hipError_t launch_attention(const FwdParams& p, Dtype dt, WorkList wl, int grid,
                            hipStream_t stream) {
    switch (dt) {
    case Dtype::BF16:
        return p.d == 64 ? launch16<__bf16, 64>(p, wl, grid, stream)
                         : launch16<__bf16, 128>(p, wl, grid, stream);
    case Dtype::FP16:
        return p.d == 64 ? launch16<_Float16, 64>(p, wl, grid, stream)
                         : launch16<_Float16, 128>(p, wl, grid, stream);
    case Dtype::FP32:
        return p.d == 64 ? launch_f32<64>(p, wl, grid, stream) : launch_f32<128>(p, wl, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace hstu
