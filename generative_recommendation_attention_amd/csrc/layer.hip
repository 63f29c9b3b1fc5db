// The HSTU layer's surroundings of the attention, on the matrix cores (bf16 /
// fp16), HSTU paper translation §3 and §3.3: f1 and f2 are one linear layer
// each, phi_1 = SiLU, Norm = layer normalisation, residual connections; the
// paper fuses phi_1(f_1(.)) into one operator and the layer norm with the
// output MLP into another.  Per token t:
//
//   layer_in:   [u | v | q | k] = silu(W1 x_t + b1)
//               (W1: (4 heads d) x d_model, row-major; each part written as
//               (T, heads, d), the layout the attention reads)
//   layer_out:  y_t = x_t + W2 (LN(a_t) * u_t) + b2
//               (W2: d_model x (heads d); LN over heads d with gamma, beta)
//
// Both are products with a small inner dimension K (d_model or heads d, at
// most 512), so each wave keeps its 32 tokens' whole K-long rows as MFMA B
// operands in registers: layer_out normalises and gates them there (the
// prologue), then both kernels stream the weight matrix through LDS in
// chunks of output features (one barrier per chunk) and apply bias, SiLU or
// residual in the epilogue.  The products are computed transposed (features
// down, tokens across), so a lane ends with one token and runs of 4
// consecutive features; each wave turns its 32 x 32 result tile around in
// LDS and stores whole 64-byte token rows (layer_out first brings the
// residual rows into that tile straight from HBM, so neither epilogue reads
// global memory).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace hstu {

namespace {

template <int K>
struct LayerCfg {
    static constexpr int NW = 4;
    static constexpr int ROWS = 32 * NW;           // tokens per workgroup
    // Output features per chunk: 32 (16-32 KB of weights).  At K = 256, 64
    // measured 3-5 % slower (one chunk of prefetch covers less time when the
    // chunk is bigger but arrives all at once).
    static constexpr int NC = 32;
    static constexpr int NB = NC / 32;             // 32-feature blocks per chunk
    static constexpr int RB = 2 * K;               // bytes of one weight row
    static constexpr int CH = RB / 16;             // 16-byte chunks per row
    static constexpr int CHUNK_BYTES = NC * RB;
    static constexpr int LOADS = CHUNK_BYTES / 1024 / NW;   // wave loads per chunk
    static constexpr int RPL = 1024 / RB;          // rows one wave load covers
    static constexpr int NKS = K / 16;             // k-steps
    static_assert(K == 128 || K == 256 || K == 512, "inner dimension");
    static_assert(LOADS * NW * 1024 == CHUNK_BYTES, "chunk must split into whole wave loads");
};

// Swizzle of a weight row's 16-byte chunks: 16 consecutive rows read at one
// logical chunk land in 16 different physical chunks.
__device__ __forceinline__ int wswz(int r) {
    return 2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1);
}

template <int K>
struct WeightStage {
    using C = LayerCfg<K>;
    int goff[C::LOADS];   // global byte offset of each of this lane's loads
    int dst[C::LOADS];    // LDS byte offset (wave-uniform part) of each load
    // LDS byte offset of row l32, logical chunk 2ks + g, for ks < 8; the
    // swizzle changes only the low 4 chunk bits, so k-step ks reads at
    // rd[ks % 8] + 256 (ks / 8).
    int rd[8];
    __device__ WeightStage(int lane, int wv) {
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int L = wv + C::NW * i;
            const int r = L * C::RPL + lane / C::CH;
            const int pc = lane % C::CH;
            goff[i] = r * C::RB + 16 * (pc ^ wswz(r));
            dst[i] = L * 1024;
        }
        const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) rd[ks] = l32 * C::RB + 16 * ((2 * ks + g) ^ wswz(l32));
    }
    // Rows [c0, c0 + NC) of the (n x K) weight matrix into `buf`; rows past n
    // read as zero.
    __device__ void issue(const uint16_t* w, int n, int c0, unsigned char* buf) const {
        const __amdgpu_buffer_rsrc_t r =
                make_rsrc32(w + (int64_t)c0 * K, min(n - c0, C::NC) * C::RB);
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) load16_to_lds(r, buf + dst[i], goff[i]);
    }
};

// The products of one chunk: acc[b] = sum_k W[c0 + 32 b + i][k] * Z[token j][k]
// (i: feature within the block, j: the lane's token).
template <typename T, int K>
__device__ __forceinline__ void chunk_products(const unsigned char* buf, const WeightStage<K>& st,
                                               const typename Mfma<T>::v8* z, f32x16* acc) {
    using C = LayerCfg<K>;
    using M = Mfma<T>;
#pragma unroll
    for (int b = 0; b < C::NB; ++b) acc[b] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
            const typename M::v8 wa = *reinterpret_cast<const typename M::v8*>(
                    buf + b * 32 * C::RB + 256 * (ks / 8) + st.rd[ks % 8]);
            acc[b] = M::mma(wa, z[ks], acc[b]);
        }
}

// Chunks [c_begin, c_end) of the weight matrix through PF + 1 LDS buffers
// (chunks c_begin .. c_begin + PF - 1 must already be issued into buffers
// 0 .. PF - 1, those past c_end as empty loads).  Iteration c waits for
// chunk c, issues chunk c + PF (an empty load past c_end, so that PF - 1
// chunks' loads always follow chunk c's), stores chunk c-1's results and
// then computes chunk c's products.  The wait counts loads only in the
// sense that matters: loads complete in issue order, so while chunk c's are
// outstanding so are the (PF - 1) * LOADS issued after them; the epilogue's
// stores, also counted, can only make it wait longer.  The epilogue must not
// read global memory (the compiler would wait for every load before it, the
// chunks in flight included).
template <typename T, int K, int PF, typename Epi>
__device__ __forceinline__ void chunk_loop(const uint16_t* w, int n, int c_begin, int c_end,
                                           const WeightStage<K>& st, unsigned char* lds,
                                           const typename Mfma<T>::v8* z, Epi& epilogue) {
    using C = LayerCfg<K>;
    constexpr int NS = PF + 1;
    f32x16 acc[C::NB], prev[C::NB];
    const int n_end = min(n, c_end * C::NC);
    for (int c = c_begin; c < c_end; ++c) {
        __builtin_amdgcn_s_waitcnt(VMCNT_LE((PF - 1) * C::LOADS));
        __syncthreads();
        const int i = c - c_begin;
        st.issue(w, n_end, (c + PF) * C::NC, lds + ((i + PF) % NS) * C::CHUNK_BYTES);
        if (c > c_begin) epilogue(c - 1, prev);
        chunk_products<T, K>(lds + (i % NS) * C::CHUNK_BYTES, st, z, acc);
#pragma unroll
        for (int b = 0; b < C::NB; ++b) prev[b] = acc[b];
    }
    __builtin_amdgcn_s_waitcnt(VMCNT_LE(0));   // (the empty loads past the end)
    if (c_begin < c_end) epilogue(c_end - 1, prev);
}

// Chunks in flight: two at K <= 256, one at K = 512 (its 32 KB chunks).
template <int K> struct LayerPf { static constexpr int value = K <= 256 ? 2 : 1; };

struct LayerInArgs {
    const uint16_t* x;
    const uint16_t* w1;
    const float* b1;
    uint16_t* out[4];   // u, v, q, k
    int64_t T;
    int heads_d;        // heads * d
    int chunks_per_wg;  // output chunks per workgroup (grid.y splits them)
};

template <typename T, int K>
__global__ __launch_bounds__(256, 2) void layer_in_kernel(LayerInArgs a) {
    using C = LayerCfg<K>;
    using M = Mfma<T>;
    using v4 = typename M::v4;
    constexpr int PF = LayerPf<K>::value;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[(PF + 1) * C::CHUNK_BYTES];
    __shared__ __attribute__((aligned(16))) float sbias[4 * 512];   // b1 (4 heads d <= 2048)
    // Per wave, a 32 x 32 tile of results on its way out: token rows of 64
    // bytes, 16-byte chunks swizzled by row so that both the writes (a lane
    // per token) and the reads (four lanes per token) spread over the banks.
    __shared__ __attribute__((aligned(16))) unsigned char tbuf[C::NW * 32 * 64];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int64_t t0 = (int64_t)blockIdx.x * C::ROWS + 32 * wv;   // the wave's first token
    const int n = 4 * a.heads_d;
    const int nchunks = n / C::NC;
    const int c_begin = blockIdx.y * a.chunks_per_wg;
    const int c_end = min(nchunks, c_begin + a.chunks_per_wg);
    const WeightStage<K> st(lane, wv);

    // The wave's 32 token rows as B operands (token l32, k = 16 ks + 8 g ..).
    typename M::v8 z[C::NKS];
    {
        const int64_t rows = a.T - t0;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(a.x + t0 * K, (rows < 0 ? 0 : rows) * C::RB);
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
            z[ks] = __builtin_bit_cast(typename M::v8,
                                       __builtin_amdgcn_raw_buffer_load_b128(
                                               r, l32 * C::RB + (16 * ks + 8 * g) * 2, 0, 0));
    }
    // b1 into LDS (the epilogue reads no global memory); the chunk loop's
    // first barrier orders these writes before any read.
    for (int i = threadIdx.x; i < n; i += 256) sbias[i] = a.b1[i];

    {
        const int n_end = min(n, c_end * C::NC);
#pragma unroll
        for (int j = 0; j < PF; ++j)
            st.issue(a.w1, n_end, (c_begin + j) * C::NC, lds + j * C::CHUNK_BYTES);
    }
    // Epilogue of chunk c: bias and SiLU in the product's layout (lane: token
    // t0 + l32, features c0 + 8 i + 4 g + (0..3)), through the wave's tile in LDS
    // (LDS operations of one wave complete in order), then stored a token row
    // of 64 bytes per four lanes.  A chunk lies inside one part (heads d is a
    // multiple of the chunk).
    static_assert(C::NB == 1, "one 32-feature block per chunk");
    unsigned char* tw = tbuf + wv * 32 * 64;
    auto tsw = [](int r, int q) { return r * 64 + 16 * (q ^ ((r >> 1) & 3)); };
    auto epilogue = [&](int c, const f32x16* acc) {
        const int c0 = c * C::NC;
        const int part = __builtin_amdgcn_readfirstlane(c0 / a.heads_d);
        uint16_t* dst = part == 0 ? a.out[0] : part == 1 ? a.out[1] : part == 2 ? a.out[2]
                                                                               : a.out[3];
        dst += (c0 - part * a.heads_d);
        const float* bias_c = sbias + c0 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 bias = *reinterpret_cast<const f32x4*>(bias_c + 8 * i);
            f32x4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float s = acc[0][4 * i + j] + bias[j];
                y[j] = s * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * s));
            }
            const v4 yv = __builtin_convertvector(y, v4);
            *reinterpret_cast<u32x2*>(tw + tsw(l32, i) + 8 * g) = __builtin_bit_cast(u32x2, yv);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * h + (lane >> 2), q = lane & 3;
            const u32x4 row = *reinterpret_cast<const u32x4*>(tw + tsw(r, q));
            if (t0 + r < a.T)
                *reinterpret_cast<u32x4*>(dst + (t0 + r) * a.heads_d + 8 * q) = row;
        }
    };
    chunk_loop<T, K, PF>(a.w1, n, c_begin, c_end, st, lds, z, epilogue);
}

struct LayerOutArgs {
    const uint16_t* attn;
    const uint16_t* u;
    const uint16_t* x;
    const float* gamma;
    const float* beta;
    const uint16_t* w2;
    const float* b2;
    uint16_t* y;
    int64_t T;
    int d_model;
    float eps;
    int chunks_per_wg;
};

// Hides the values of z from the optimiser (no instruction is emitted).
template <int N, typename V>
__device__ __forceinline__ void opaque_n(V* z) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        u32x4 w = __builtin_bit_cast(u32x4, z[i]);
        asm volatile("" : "+v"(w));
        z[i] = __builtin_bit_cast(V, w);
    }
}

template <typename T, int K>
__global__ __launch_bounds__(256, 2) void layer_out_kernel(LayerOutArgs a) {
    using C = LayerCfg<K>;
    using M = Mfma<T>;
    using v8 = typename M::v8;
    using v4 = typename M::v4;
    typedef float f32x8v __attribute__((ext_vector_type(8)));
    constexpr int PF = LayerPf<K>::value;
    constexpr int NS = PF + 1;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[NS * C::CHUNK_BYTES];
    __shared__ __attribute__((aligned(16))) float sbias[512];   // b2 (d_model <= 512)
    // Per wave, the chunk's residual rows (32 tokens x 64 bytes, loaded
    // straight from HBM), overwritten by the results on their way out.
    __shared__ __attribute__((aligned(16))) unsigned char xt[C::NW * 2048];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, l32 = lane & 31;
    const int64_t t0 = (int64_t)blockIdx.x * C::ROWS + 32 * wv;
    const int n = a.d_model;
    const int nchunks = n / C::NC;
    const int c_begin = blockIdx.y * a.chunks_per_wg;
    const int c_end = min(nchunks, c_begin + a.chunks_per_wg);
    const int n_end = min(n, c_end * C::NC);
    const WeightStage<K> st(lane, wv);
    // (b2 first: its loads are waited for before the LDS writes)
    for (int i = threadIdx.x; i < n; i += 256) sbias[i] = a.b2[i];
#pragma unroll
    for (int j = 0; j < PF; ++j)   // (overlaps the prologue)
        st.issue(a.w2, n_end, (c_begin + j) * C::NC, lds + j * C::CHUNK_BYTES);

    // Prologue: the attention rows of the wave's 32 tokens (token l32,
    // features 16 ks + 8 g ..), normalised over all K features (the lane and
    // its partner lane ^ 32 hold one token's features between them), scaled,
    // shifted and gated by u, rounded to T: the B operands of the product.
    v8 z[C::NKS];
    auto opaque = [](v8* zz) { opaque_n<C::NKS>(zz); };
    const int64_t rows = a.T - t0;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.attn + t0 * K, (rows < 0 ? 0 : rows) * C::RB);
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.u + t0 * K, (rows < 0 ? 0 : rows) * C::RB);
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
        z[ks] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(
                                               ra, l32 * C::RB + (16 * ks + 8 * g) * 2, 0, 0));
    float sum = 0.0f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += (float)z[ks][e];
    sum += __shfl_xor(sum, 32);
    const float mean = sum * (1.0f / K);
    // (each pass widens the stored values again: kept widened across the
    // passes they would take twice the registers)
    opaque(z);
    float sq = 0.0f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float dlt = (float)z[ks][e] - mean;
            sq += dlt * dlt;
        }
    sq += __shfl_xor(sq, 32);
    opaque(z);
    const float rstd = __builtin_amdgcn_rsqf(sq * (1.0f / K) + a.eps);
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
        const int k0 = 16 * ks + 8 * g;
        const v8 uu = __builtin_bit_cast(
                v8, __builtin_amdgcn_raw_buffer_load_b128(ru, l32 * C::RB + k0 * 2, 0, 0));
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(a.gamma + k0);
        const f32x4 g1 = *reinterpret_cast<const f32x4*>(a.gamma + k0 + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4*>(a.beta + k0);
        const f32x4 b1 = *reinterpret_cast<const f32x4*>(a.beta + k0 + 4);
        f32x8v zz;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gm = e < 4 ? g0[e] : g1[e - 4];
            const float bt = e < 4 ? b0[e] : b1[e - 4];
            zz[e] = (((float)z[ks][e] - mean) * rstd * gm + bt) * (float)uu[e];
        }
        z[ks] = __builtin_convertvector(zz, v8);
    }

    // Chunk c's residual rows into the wave's tile: lane l brings 16 bytes of
    // token row 16 i + l / 4 (rows past T read as zero).
    unsigned char* xw = xt + wv * 2048;
    const int64_t rows_left = a.T - t0;
    const __amdgpu_buffer_rsrc_t rx =
            make_rsrc(a.x + t0 * n, (rows_left < 0 ? 0 : rows_left) * n * 2);
    auto issue_x = [&](int c) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            load16_to_lds(rx, xw + 1024 * i, (16 * i + (lane >> 2)) * n * 2 + c * 64 + 16 * (lane & 3));
    };
    // Epilogue of chunk c: residual and bias in the product's layout (lane:
    // token t0 + l32, features 8 i + 4 g + (0..3)), written over the residual
    // in the tile (LDS operations of one wave complete in order), then stored
    // a token row of 64 bytes per four lanes.
    static_assert(C::NB == 1, "one 32-feature block per chunk");
    auto epilogue = [&](int c, const f32x16* acc) {
        const int c0 = c * C::NC;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            unsigned char* px = xw + l32 * 64 + 16 * i + 8 * g;
            const f32x4 bias = *reinterpret_cast<const f32x4*>(sbias + c0 + 8 * i + 4 * g);
            const v4 xr = __builtin_bit_cast(v4, *reinterpret_cast<const u32x2*>(px));
            f32x4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = acc[0][4 * i + j] + bias[j] + (float)xr[j];
            *reinterpret_cast<u32x2*>(px) = __builtin_bit_cast(u32x2, __builtin_convertvector(y, v4));
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * h + (lane >> 2), q = lane & 3;
            const u32x4 row = *reinterpret_cast<const u32x4*>(xw + r * 64 + 16 * q);
            if (t0 + r < a.T) *reinterpret_cast<u32x4*>(a.y + (t0 + r) * n + c0 + 8 * q) = row;
        }
    };
    // Iteration c waits for weight chunk c and the residual of chunk c - 1,
    // finishes chunk c - 1, brings chunk c's residual into the tile just
    // freed, issues weight chunk c + PF (empty past c_end) and computes chunk
    // c's products.  Per iteration x(c) is issued before w(c + PF), so the
    // loads that may still fly at the wait are w(c + PF - 1)'s (PF = 2) or
    // none (PF = 1); loads complete in issue order, and the stores counted
    // with them can only make the wait longer.
    f32x16 acc[C::NB], prev[C::NB];
    for (int c = c_begin; c < c_end; ++c) {
        __builtin_amdgcn_s_waitcnt(VMCNT_LE(PF == 1 ? 0 : C::LOADS));
        __syncthreads();
        const int i = c - c_begin;
        if (c > c_begin) epilogue(c - 1, prev);
        // (the tile's LDS reads done before the next residual lands in it:
        // lgkmcnt 0, the other counters left open)
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));
        issue_x(c);
        st.issue(a.w2, n_end, (c + PF) * C::NC, lds + ((i + PF) % NS) * C::CHUNK_BYTES);
        chunk_products<T, K>(lds + (i % NS) * C::CHUNK_BYTES, st, z, acc);
#pragma unroll
        for (int b = 0; b < C::NB; ++b) prev[b] = acc[b];
    }
    __builtin_amdgcn_s_waitcnt(VMCNT_LE(0));
    if (c_begin < c_end) epilogue(c_end - 1, prev);
}

// Splits the output chunks over grid.y so that the launch has at least two
// workgroups per compute unit.
int chunks_per_wg(int64_t m_tiles, int nchunks) {
    const int64_t want = 2LL * device_cus();
    int split = (int)((want + m_tiles - 1) / m_tiles);
    split = split < 1 ? 1 : (split > nchunks ? nchunks : split);
    return (nchunks + split - 1) / split;
}

template <typename T, int K>
hipError_t layer_in_typed(const LayerParams& p, hipStream_t stream) {
    using C = LayerCfg<K>;
    LayerInArgs a;
    a.x = static_cast<const uint16_t*>(p.x);
    a.w1 = static_cast<const uint16_t*>(p.w1);
    a.b1 = p.b1;
    for (int i = 0; i < 4; ++i) a.out[i] = static_cast<uint16_t*>(p.uvqk[i]);
    a.T = p.T;
    a.heads_d = p.heads_d;
    const int64_t m_tiles = (p.T + C::ROWS - 1) / C::ROWS;
    const int nchunks = 4 * p.heads_d / C::NC;
    a.chunks_per_wg = chunks_per_wg(m_tiles, nchunks);
    const dim3 grid((unsigned)m_tiles, (unsigned)((nchunks + a.chunks_per_wg - 1) / a.chunks_per_wg));
    hipLaunchKernelGGL((layer_in_kernel<T, K>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int K>
hipError_t layer_out_typed(const LayerParams& p, hipStream_t stream) {
    using C = LayerCfg<K>;
    LayerOutArgs a;
    a.attn = static_cast<const uint16_t*>(p.attn);
    a.u = static_cast<const uint16_t*>(p.u);
    a.x = static_cast<const uint16_t*>(p.x);
    a.gamma = p.gamma;
    a.beta = p.beta;
    a.w2 = static_cast<const uint16_t*>(p.w2);
    a.b2 = p.b2;
    a.y = static_cast<uint16_t*>(p.y);
    a.T = p.T;
    a.d_model = p.d_model;
    a.eps = p.eps;
    const int64_t m_tiles = (p.T + C::ROWS - 1) / C::ROWS;
    const int nchunks = p.d_model / C::NC;
    a.chunks_per_wg = chunks_per_wg(m_tiles, nchunks);
    const dim3 grid((unsigned)m_tiles, (unsigned)((nchunks + a.chunks_per_wg - 1) / a.chunks_per_wg));
    hipLaunchKernelGGL((layer_out_kernel<T, K>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t layer_in_k(const LayerParams& p, hipStream_t s) {
    switch (p.d_model) {
    case 128: return layer_in_typed<T, 128>(p, s);
    case 256: return layer_in_typed<T, 256>(p, s);
    case 512: return layer_in_typed<T, 512>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t layer_out_k(const LayerParams& p, hipStream_t s) {
    switch (p.heads_d) {
    case 128: return layer_out_typed<T, 128>(p, s);
    case 256: return layer_out_typed<T, 256>(p, s);
    case 512: return layer_out_typed<T, 512>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_layer_in(const LayerParams& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return layer_in_k<__bf16>(p, stream);
    if (dt == Dtype::FP16) return layer_in_k<_Float16>(p, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_layer_out(const LayerParams& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return layer_out_k<__bf16>(p, stream);
    if (dt == Dtype::FP16) return layer_out_k<_Float16>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace hstu
