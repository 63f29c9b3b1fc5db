// HSTU jagged attention backward on gfx950 matrix cores (bf16 / fp16).
//
// Forward, per sequence and head:  out[r] = (1/n) sum_{c seen by r} silu(x_rc) v_c,
// x_rc = alpha <q_r, k_c>.  For an upstream gradient dO, per kept pair (r, c):
//
//   dv_c += silu(x_rc) / n * dO_r
//   g_rc  = (alpha / n) * silu'(x_rc) * <dO_r, v_c>,  silu'(x) = sig(x) (1 + x (1 - sig(x)))
//   dq_r += g_rc * k_c,        dk_c += g_rc * q_r
//
// The pages give only the idea: the backward recomputes the attention block by
// block instead of storing the h x N x N tensor, and accumulates gradients on
// chip (HSTU paper translation, Appendix G).  Here two kernels, so that no
// gradient is accumulated with atomics:
//
//   attn_bwd_dkv: a work item is (sequence, head, 128-key tile); each wave
//     keeps 32 keys' K and V in registers and the dK, dV accumulators for them,
//     and streams the 32-row query blocks at or below its keys (Q and dO staged
//     in LDS):  S = Q K^T and dP = dO V^T (keys across, queries down), then
//     P = silu(alpha S) and dS = dP * silu'(alpha S) in registers, then
//     dV^T += dO^T P and dK^T += Q^T dS (the contraction over queries takes P
//     and dS straight from the accumulators; dO^T and Q^T come from gfx950's
//     transposing LDS read, as V^T does in the forward).
//   attn_bwd_dq: a work item is (sequence, head, 128-query tile); each wave
//     keeps 32 queries' Q and dO in registers and streams the 32-key blocks up
//     to its diagonal (K and V staged in LDS): S^T = K Q^T and dP^T = V dO^T,
//     dS^T in registers, dQ^T += K^T dS^T.
//
// S and dP are recomputed by both kernels (seven block products per kept
// block pair instead of five) in exchange for no atomics and no fp32 dQ
// buffer.  The 1/n and alpha/n factors are applied once, in the epilogues.
//
// Tiles in LDS: 32 rows per block, 16-byte chunks XOR-swizzled per row; an
// operand read both ways (row reads and transposing reads) is staged twice,
// once in each swizzle, so neither read pattern has bank conflicts.  PF + 1
// slots (PF = 1): block c+1 streams in (straight from HBM into LDS) while
// block c is consumed; one barrier per block.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "internal.h"
#include "schedule.h"

namespace hstu {

namespace {

constexpr float BWD_LOG2E = 1.4426950408889634f;

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    const int32_t* offsets;
    const int32_t* ntgt;   // candidates per sequence (target-aware mask), or null
    WorkList wl;
    // (T, heads, D) jagged: rows heads * D apart, heads D apart; dense
    // (B, heads, S, D): rows D apart, heads S * D apart (offsets i * S)
    int64_t row_stride;
    int64_t head_stride;
    int num_seqs;
    int heads;
    float score_scale;   // -alpha log2(e): the S operand's scale (K in dK/dV, Q in dQ)
    float dv_scale;      // 1 / n
    float g_scale;       // alpha / n
};

// Relative attention bias (the forward's reading: rab(r, c) = wpos[r - c] +
// wtime[bucket(ts_r - ts_c)], added to alpha <q_r, k_c> before SiLU).  Both
// kernels recompute it and start the score accumulators at -log2(e) rab (the
// scores being -log2(e) alpha s, from the pre-scaled operand); the
// dQ kernel, which holds one query per lane and 16 keys per lane in registers,
// also sums each kept pair's score gradient into the two tables' gradients.
// (A separate argument type, so that the other kernels keep their argument
// block.)
struct BwdArgsRab : BwdArgs {
    const int32_t* ts;     // token timestamps
    const float* wpos;
    const float* wtime;
    float* gpart;          // [nparts][gstride] table-gradient partials: npos entries, then 32
    int npos;
    int ntime;
    int gstride;
    int nparts;
    float bias_scale;      // -log2(e)
};
template <bool RAB> struct BwdArgsOf { using type = BwdArgs; };
template <> struct BwdArgsOf<true> { using type = BwdArgsRab; };

// Bias staging per slot: the timestamps of the block's 32 streamed rows (64
// words: one wave load), then RABB_WIN entries of wpos, the distances the
// block's pairs with the item's 128 rows can take.
constexpr int RABB_TS = 64;
constexpr int RABB_WIN = 192;
constexpr int RABB_WORDS = RABB_TS + RABB_WIN;

// Time table by v_ffbh_u32(gap + 1) + 1 (index 0: a zero argument, gap -1),
// already capped at the last bucket, as the forward keeps it.
__device__ __forceinline__ int rab_time_bucket(int idx, int ntime) {
    return idx == 0 ? ntime - 1 : min(32 - idx, ntime - 1);
}

__device__ __forceinline__ int ffbh_u32(uint32_t x) {
    int f;
    asm("v_ffbh_u32 %0, %1" : "=v"(f) : "v"(x));
    return f;
}

// Wave-wide minimum / maximum (every lane takes part; the result is uniform).
// Minimum / maximum over the wave without LDS: within each 16-lane row by
// DPP (quad permutations xor 1 and xor 2, then the half-row and row mirrors,
// which pair each quad and then each half-row with the other), then the four
// rows' results read out to scalars.  Every lane must be active.
template <bool MAX>
__device__ __forceinline__ int wave_reduce_i32(int x) {
    auto op = [](int u, int v) { return MAX ? max(u, v) : min(u, v); };
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));    // quad xor 1
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));    // quad xor 2
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));   // row half mirror
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));   // row mirror
    return op(op(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
              op(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
__device__ __forceinline__ int wave_min_i32(int x) { return wave_reduce_i32<false>(x); }
__device__ __forceinline__ int wave_max_i32(int x) { return wave_reduce_i32<true>(x); }

// Blocks whose every pair lies in the last time bucket (the latest key at
// least 2^(ntime-1) - 1 before the earliest query) take the time term as one
// constant, the last bucket's entry, instead of a per-pair lookup: the same
// values, since every such pair's capped bucket is the last one.  At d = 64
// only: at d = 128 the second path costs the bias kernels 12-20 more
// spilled registers.
__device__ __forceinline__ bool rab_far(int rmin, int kmax, int ntime) {
    return (int64_t)rmin - kmax >= ((int64_t)1 << (ntime - 1)) - 1;
}

// Sum of each of a lane's 16 registers over the 32 lanes of its half-wave,
// by recursive halving (four exchanges that each halve the registers a lane
// carries, then one that completes the sum): lane l ends with the sum of
// register (l >> 1) & 15.  The exchanges run on the vector ALUs, not through
// LDS: partners l ^ 16 by v_permlane16_swap (which swaps the odd 16-lane rows
// of one register with the even rows of another, so each lane of a row pair
// ends with its own half and its partner's, no select needed), then l ^ 15,
// l ^ 7, l ^ 2 and l ^ 1 by DPP (row mirror, half-row mirror, two quad
// permutations).  Those partners differ from l in bit 3, 2, 1 and 0 in turn,
// and together with 16 they reach all 32 lanes, so every lane's total covers
// its half-wave.
template <int CTRL>
__device__ __forceinline__ float dpp_f32c(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                             0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float half_wave_column_sum(const f32x16& x, int l32) {
    constexpr int ROW_MIRROR = 0x140, ROW_HALF_MIRROR = 0x141;
    constexpr int QUAD_XOR2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);
    constexpr int QUAD_XOR1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);
    const bool b3 = l32 & 8, b2 = l32 & 4, b1 = l32 & 2;
    float y[8], z[4], w[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // (vector elements copied to scalars first: __builtin_bit_cast of an
        // element of a vector-typed value reads element 0 with this compiler)
        const float lo = x[i], hi = x[i + 8];
        const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, lo),
                                                         __builtin_bit_cast(unsigned, hi), false,
                                                         false);
        const unsigned r0 = r[0], r1 = r[1];
        y[i] = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        z[i] = (b3 ? y[i + 4] : y[i]) + dpp_f32c<ROW_MIRROR>(b3 ? y[i] : y[i + 4]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        w[i] = (b2 ? z[i + 2] : z[i]) + dpp_f32c<ROW_HALF_MIRROR>(b2 ? z[i] : z[i + 2]);
    const float u = (b1 ? w[1] : w[0]) + dpp_f32c<QUAD_XOR2>(b1 ? w[0] : w[1]);
    return u + dpp_f32c<QUAD_XOR1>(u);
}

// One register's share of the diagonal sums of a 32 x 32 score block, on the
// vector ALUs.  Lane (g, l) holds query l and, in register r, key
// S + 4g with S = 8(r/4) + r%4.  Both half-waves take the same pattern, as if
// their key were S: dhi[l] += x[l + S] (no wrap) and dlo[l] += x[l + S - 32]
// (wrap), within the half-wave; the second half's real key is 4 further, so
// its sums sit 4 distances lower, which the combine below accounts for.  A
// 32-lane shift is a row shift (DPP) for the part within a 16-lane row and,
// for the part crossing into the other row, a row shift of the other row's
// values, which one v_permlane16_swap of the register with itself provides
// (op holds the even row's values in the odd rows, sp the odd row's in the
// even rows); row masks send each part to dhi or dlo.
// acc += src moved by a DPP pattern, in the rows of a row mask only (the
// other rows keep acc: a DPP add leaves the lanes of disabled rows
// unwritten).  One instruction; the compiler's own form was a DPP move into
// a zeroed register and an add.  (The s_nop covers the wait states a DPP read
// needs after the instruction that wrote its source.)
#define HSTU_ADD_DPP(acc, src, pattern, rows)                                             \
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %0 " pattern " row_mask:" rows                \
        " bank_mask:0xf bound_ctrl:1"                                                      \
        : "+v"(acc)                                                                        \
        : "v"(src))
#define HSTU_ROW_SHL(n) "row_shl:" #n
#define HSTU_ROW_SHR(n) "row_shr:" #n
template <int R>
__device__ __forceinline__ void diag_step(float x, float& dhi, float& dlo) {
    constexpr int S = 8 * (R >> 2) + (R & 3);
    if constexpr (S == 0) {
        dhi += x;
        return;
    }
    const unsigned xu = __builtin_bit_cast(unsigned, x);
    const auto sw = __builtin_amdgcn_permlane16_swap(xu, xu, false, false);
    const unsigned opu = sw[0], spu = sw[1];
    const float op = __builtin_bit_cast(float, opu), sp = __builtin_bit_cast(float, spu);
    // S < 16: dhi += row_shl:S(x) (all rows), dhi += row_shr:16-S(sp) (even
    // rows), dlo += row_shr:16-S(op) (odd rows).  S = 16 + B: dhi +=
    // row_shl:B(sp) (even rows), dlo += row_shl:B(op) (odd rows), dlo +=
    // row_shr:16-B(x) (all rows); B = 0 moves sp and op unshifted.
#define HSTU_DIAG_LO(s, r16)                                                                \
    if constexpr (S == s) {                                                                \
        HSTU_ADD_DPP(dhi, x, HSTU_ROW_SHL(s), "0xf");                                     \
        HSTU_ADD_DPP(dhi, sp, HSTU_ROW_SHR(r16), "0x5");                                  \
        HSTU_ADD_DPP(dlo, op, HSTU_ROW_SHR(r16), "0xa");                                  \
    }
#define HSTU_DIAG_HI(s, b, r16)                                                             \
    if constexpr (S == s) {                                                                \
        HSTU_ADD_DPP(dhi, sp, HSTU_ROW_SHL(b), "0x5");                                    \
        HSTU_ADD_DPP(dlo, op, HSTU_ROW_SHL(b), "0xa");                                    \
        HSTU_ADD_DPP(dlo, x, HSTU_ROW_SHR(r16), "0xf");                                   \
    }
    HSTU_DIAG_LO(1, 15) HSTU_DIAG_LO(2, 14) HSTU_DIAG_LO(3, 13)
    HSTU_DIAG_LO(8, 8) HSTU_DIAG_LO(9, 7) HSTU_DIAG_LO(10, 6) HSTU_DIAG_LO(11, 5)
    if constexpr (S == 16) {
        HSTU_ADD_DPP(dhi, sp, "quad_perm:[0,1,2,3]", "0x5");
        HSTU_ADD_DPP(dlo, op, "quad_perm:[0,1,2,3]", "0xa");
    }
    HSTU_DIAG_HI(17, 1, 15) HSTU_DIAG_HI(18, 2, 14) HSTU_DIAG_HI(19, 3, 13)
    HSTU_DIAG_HI(24, 8, 8) HSTU_DIAG_HI(25, 9, 7) HSTU_DIAG_HI(26, 10, 6) HSTU_DIAG_HI(27, 11, 5)
#undef HSTU_DIAG_LO
#undef HSTU_DIAG_HI
}
#undef HSTU_ROW_SHL
#undef HSTU_ROW_SHR
#undef HSTU_ADD_DPP
template <int... Rs>
__device__ __forceinline__ void diag_steps(const f32x16& d, float& dhi, float& dlo,
                                           std::integer_sequence<int, Rs...>) {
    (diag_step<Rs>(static_cast<float>(d[Rs]), dhi, dlo), ...);
}

// Shapes shared by both kernels: 4 waves of 32 rows (128 rows per item), 32-row
// streamed blocks.
template <int D>
struct BwdCfg {
    static constexpr int NW = 4;
    static constexpr int ROWS = 32 * NW;              // rows per item
    static constexpr int RB = 2 * D;                  // bytes per row in LDS
    static constexpr int CH = RB / 16;                // 16-byte chunks per row
    static constexpr int ARR = 32 * RB;               // one 32-row array in LDS
    static constexpr int RPL = 1024 / RB;             // rows one wave load covers
    static constexpr int LPA = ARR / 1024 / NW;       // wave loads per array
    static constexpr int NKS = D / 16;                // k-steps over the head dim
    static constexpr int NDB = D / 32;                // 32-wide head-dim blocks
    // Blocks staged ahead.  (Two at d = 64 measured slower: 0.80 ms instead of
    // 0.69 ms for the dK/dV + dQ pair at 16 x 4096; again with the loads the
    // compiler does not track: 0.612 -> 0.640 ms with two in the dK/dV kernel
    // only, 0.690 with two in both, whose dQ kernel then needs 180 VGPRs and
    // loses its third workgroup per CU.)
    static constexpr int PF = 1;
    static_assert(LPA * NW * 1024 == ARR, "array must split into whole wave loads");
};

// Per-lane pieces of the staging and operand addresses (see the forward).
template <int D>
struct LaneOffsets {
    using C = BwdCfg<D>;
    int gk[C::LPA], gv[C::LPA];   // global byte offsets of this lane's loads (row-read, transposed swizzle)
    int dst[C::LPA];              // LDS byte offset of each load inside an array
    int rowrd[C::NKS];            // row read of row l32, k-step ks (= rowrd[0] ^ 32 ks)
    int tr_lo[C::NDB], tr_hi[C::NDB];   // transposing reads, head-dim block db
    __device__ LaneOffsets(int lane, int wv, int row_bytes) {
        constexpr int CH = C::CH;
#pragma unroll
        for (int i = 0; i < C::LPA; ++i) {
            const int L = wv + C::NW * i;
            const int r = L * C::RPL + lane / CH;
            const int pc = lane % CH;
            gk[i] = r * row_bytes + 16 * (pc ^ kswz<CH>(r));
            gv[i] = r * row_bytes + 16 * (pc ^ vswz<CH>(r));
            dst[i] = L * 1024;
        }
        const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) rowrd[ks] = l32 * C::RB + 16 * ((2 * ks + g) ^ kswz<CH>(l32));
        const int v_row = 4 * g + ((lane & 15) >> 2);
        const int v_colb = 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const int cb = 64 * db + v_colb;
            tr_lo[db] = v_row * C::RB + 16 * ((cb >> 4) ^ vswz<CH>(v_row)) + (cb & 15);
            tr_hi[db] = (v_row + 8) * C::RB + 16 * ((cb >> 4) ^ vswz<CH>(v_row + 8)) + (cb & 15);
        }
    }
};

// The row-read offsets of a block's k-steps.  (2 ks + g) ^ swizzle =
// 2 ks ^ (g ^ swizzle), so k-step ks's offset is k-step 0's XOR 32 ks (the
// row's base has no bits below the row size).  At d = 128 the eight offsets
// held across the block loop pushed other values to scratch, whose reloads
// inside the loop waited for the prefetched tiles too; there the offsets are
// rebuilt from k-step 0's per block (an empty asm makes that value new in
// each block, so the compiler does not hoist the XORs back out).
template <int D>
struct RowReads {
    int r[BwdCfg<D>::NKS];
    __device__ __forceinline__ explicit RowReads(const LaneOffsets<D>& lo) {
        if constexpr (D == 128) {
            int r0 = lo.rowrd[0];
            asm volatile("" : "+v"(r0));
#pragma unroll
            for (int ks = 0; ks < BwdCfg<D>::NKS; ++ks) r[ks] = r0 ^ (32 * ks);
        } else {
#pragma unroll
            for (int ks = 0; ks < BwdCfg<D>::NKS; ++ks) r[ks] = lo.rowrd[ks];
        }
    }
};

// Stages 32 rows of one tensor (rows [row0, row0 + 32) of a sequence whose
// first row is at `base`) into an LDS array, in the row-read swizzle (tr =
// false) or the transposing-read swizzle (tr = true).  Rows at or past
// `rows_avail` read as zero.
template <int D>
__device__ __forceinline__ void stage(const uint16_t* base, int64_t row_stride, int row0,
                                      int rows_avail, int row_bytes, unsigned char* arr,
                                      const LaneOffsets<D>& lo, bool tr) {
    const int n = min(rows_avail - row0, 32);
    const __amdgpu_buffer_rsrc_t r =
            make_rsrc32(base + (int64_t)row0 * row_stride, n * row_bytes);
#pragma unroll
    for (int i = 0; i < BwdCfg<D>::LPA; ++i)
        load16_to_lds(r, arr + lo.dst[i], tr ? lo.gv[i] : lo.gk[i]);
}

template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::v8 row_read(const unsigned char* arr, int off) {
    return *reinterpret_cast<const typename Mfma<T>::v8*>(arr + off);
}

template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::v8 tr_read(const unsigned char* arr, int t,
                                                        const LaneOffsets<D>& lo, int db) {
    const unsigned char* p = arr + 16 * t * BwdCfg<D>::RB;
    const i16x4 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(p + lo.tr_lo[db]));
    const i16x4 b = lds_read_tr16(reinterpret_cast<const uint16_t*>(p + lo.tr_hi[db]));
    return __builtin_bit_cast(typename Mfma<T>::v8,
                              __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 32 rows x D of a row-major tensor as the B operand of the row-by-head-dim
// product (lane: row l32, head-dim slice 16ks + 8g .. +8); rows past the
// range read as zero.
template <typename T, int D>
__device__ __forceinline__ void load_rows_b(const uint16_t* base, int64_t row_stride, int rows,
                                            int row_bytes, int l32, int g,
                                            typename Mfma<T>::v8* op) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (int64_t)rows * row_bytes);
#pragma unroll
    for (int ks = 0; ks < BwdCfg<D>::NKS; ++ks)
        op[ks] = __builtin_bit_cast(typename Mfma<T>::v8,
                                    __builtin_amdgcn_raw_buffer_load_b128(
                                            r, l32 * row_bytes + (ks * 16 + g * 8) * 2, 0, 0));
}

// P and dS for one accumulator register: x = alpha s, sig = 1/(1 + e^-x),
// p = silu(x) = x sig, and silu'(x) = sig (1 + x (1 - sig)) = sig + p (1 - sig),
// so ds = dp * fma(p, 1 - sig, sig): one multiply fewer than the first form.
__device__ __forceinline__ void pointwise(float s, float dp, float alpha, float* p, float* ds) {
    const float x = alpha * s;
    const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-BWD_LOG2E * x));
    const float pr = x * sig;
    *p = pr;
    *ds = dp * __builtin_fmaf(pr, 1.0f - sig, sig);
}

// The same from m = -log2(e) x, the score of an operand pre-scaled by
// -alpha log2(e) (the 16-bit kernels): sig = 1/(1 + 2^m), and with x =
// -ln(2) m the weight comes out divided by -ln(2), p' = m sig (the dV
// epilogue multiplies the -ln(2) back in), while ds = dp (sig + p (1 - sig))
// = dp fma(p', ln(2) (sig - 1), sig).
constexpr float BWD_LN2 = 0.69314718055994531f;
__device__ __forceinline__ void pointwise_m(float m, float dp, float* p, float* ds) {
    const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(m));
    const float pr = m * sig;
    *p = pr;
    *ds = dp * __builtin_fmaf(pr, __builtin_fmaf(sig, BWD_LN2, -BWD_LN2), sig);
}

// Writes a transposed accumulator (head-dim rows x 32 tokens: lane = token
// l32, registers = head-dim rows 32db + 8(r/4) + 4g + r%4) scaled, rounded to
// T; tokens at or past `rows` are dropped.
template <typename T, int D>
__device__ __forceinline__ void store_rows(uint16_t* base, int rows, int row_bytes, int l32, int g,
                                           const f32x16* acc, float scale) {
    using v4 = typename Mfma<T>::v4;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, (int64_t)rows * row_bytes);
#pragma unroll
    for (int db = 0; db < BwdCfg<D>::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = acc[db][4 * i + j] * scale;
            const v4 y = __builtin_convertvector(x, v4);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, y), r,
                                                  l32 * row_bytes + (db * 32 + 8 * i + 4 * g) * 2,
                                                  0, 0);
        }
}

// ---------------------------------------------------------------------------
// dK, dV.  Item (sequence, head, key tile kt): keys [128 kt, 128 kt + 128).
// Wave wv owns keys kw0 .. kw0 + 31, kw0 = 128 kt + 32 wv; query block j
// (rows 32 j .. 32 j + 31) is streamed for j from 4 kt on.  For the wave, a
// block below its keys is skipped, the block on its diagonal (and, with the
// target-aware mask, any block when its keys reach the candidates) is masked,
// and the rest are full.  LDS slot: Q (row reads), Q (transposed), dO (row
// reads), dO (transposed).
// ---------------------------------------------------------------------------
// Three workgroups per CU (at most 168 VGPRs) at d = 64: the plain kernels fit
// without spills (0.616 -> 0.605 ms for the backward at 16 x 4096), the bias
// forms spill none (causal) or a few outside the block loop (causal: 0.933 -> 0.865
// ms for its backward at 16 x 4096; under the target-aware mask 1.503 ->
// 1.403 ms at 16 x (3072 + 1024)).  At d = 128 two.
template <typename T, int D, bool FUSED, bool TGT, bool RAB = false>
__global__ __launch_bounds__(256, (D == 64) ? 3 : 2) void attn_bwd_dkv(
        typename BwdArgsOf<RAB>::type a) {
    using C = BwdCfg<D>;
    using M = Mfma<T>;
    using v8 = typename M::v8;
    constexpr int SLOT = 4 * C::ARR;
    constexpr int PF = C::PF, NS = PF + 1;
    constexpr int LT = 4 * C::LPA;   // loads per wave per block
    constexpr int RAB_BYTES = RAB ? NS * RABB_WORDS * 4 : 0;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[NS * SLOT + RAB_BYTES];
    __shared__ int s_item[NQ];
    __shared__ LocalTables lt;
    __shared__ float ttab[RAB ? 33 : 1];   // time term by v_ffbh_u32(gap + 1) + 1, times -log2(e)
    static_assert(C::NW * 64 >= FUSE_SEQS && C::NW * 64 >= 32 * NQ, "fused tables need a thread per sequence");
    static_assert(NS * SLOT + RAB_BYTES + (int)sizeof(LocalTables) <= 80 * 1024,
                  "LDS for two workgroups per CU");
    static_assert(!RAB || PF == 1, "bias: one block ahead");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = a.row_stride;
    const int row_bytes = (int)(row_stride * 2);
    const LaneOffsets<D> lo(lane, wv, row_bytes);
    if constexpr (RAB) {
        if (tid < 33) ttab[tid] = a.wtime[rab_time_bucket(tid, a.ntime)] * a.bias_scale;
    }

    Tables tb;
    if constexpr (FUSED)
        tb = build_local_tables(lt, reinterpret_cast<int*>(lds), a.offsets, a.num_seqs, H, C::ROWS,
                                a.wl.ctl);
    else
        tb = global_tables(a.wl);
    clear_sets(a.wl.ctl, a.wl.set + 2, 1);   // (the next call's sets: see the launcher)
    ItemSource src(a.wl.ctl, a.wl.set);
    int qx, w;
    while (src.next(tb, s_item, &qx, &w)) {
        const Item it = decode_item(tb, a.num_seqs, H, qx, w);
        const int seq = __builtin_amdgcn_readfirstlane(it.seq);
        const int head = __builtin_amdgcn_readfirstlane(it.head);
        const int start = __builtin_amdgcn_readfirstlane(a.offsets[seq]);
        const int s = __builtin_amdgcn_readfirstlane(a.offsets[seq + 1]) - start;
        const int ntile = (s + C::ROWS - 1) / C::ROWS;
        const int kt = ntile - 1 - __builtin_amdgcn_readfirstlane(it.qtile);   // costliest first
        int hist = s;
        if constexpr (TGT) hist = s - min(max(__builtin_amdgcn_readfirstlane(a.ntgt[seq]), 0), s);
        const int k0i = kt * C::ROWS;
        const int kw0 = k0i + 32 * wv;
        const bool live = kw0 < s;
        // Query blocks: from the item's first key to the sequence end; when
        // every key of the item is a candidate, only its own rows see them.
        const int q_end = (TGT && k0i >= hist) ? min(s, k0i + C::ROWS) : s;
        const int j0 = k0i / 32;
        const int nblk = (q_end + 31) / 32 - j0;
        const int64_t seq_base = (int64_t)start * H * D + (int64_t)head * a.head_stride;
        const uint16_t* qb = a.q + seq_base;
        const uint16_t* ob = a.dout + seq_base;

        v8 kop[C::NKS], vop[C::NKS];
        load_rows_b<T, D>(a.k + seq_base + (int64_t)kw0 * row_stride, row_stride, s - kw0,
                          row_bytes, l32, g, kop);
        load_rows_b<T, D>(a.v + seq_base + (int64_t)kw0 * row_stride, row_stride, s - kw0,
                          row_bytes, l32, g, vop);
        // K * (-alpha log2(e)), rounded to T (nearest even): S^T then holds
        // m = -log2(e) alpha s, the exponent the pointwise pass needs.
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
            kop[ks] = __builtin_convertvector(
                    __builtin_convertvector(kop[ks], f32x8) * a.score_scale, v8);
        f32x16 dk[C::NDB], dv[C::NDB];
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) dk[db] = dv[db] = (f32x16){};
        // With the bias: 1 - ts of this lane's key, so that ts_q + c1 = gap + 1.
        uint32_t c1 = 0;
        int kmax = 0;   // the wave's latest key timestamp
        // Target-aware mask: a candidate row sits right after the history, so
        // its position term is wpos[hist - key] for this lane's history key
        // (pos_c) and wpos[0] for its own key (pos_0).
        float pos_c = 0.0f, pos_0 = 0.0f;
        if constexpr (RAB) {
            c1 = 1u - __builtin_amdgcn_raw_buffer_load_b32(
                              make_rsrc(a.ts + start + kw0, (int64_t)(s - kw0) * 4), l32 * 4, 0, 0);
            if constexpr (D == 64)
                kmax = wave_max_i32(kw0 + l32 < s ? (int)(1u - c1) : INT32_MIN);
            if constexpr (TGT) {
                const int dc = hist - (kw0 + l32);
                const float w = a.wpos[min(max(dc, 0), a.npos - 1)];
                pos_c = (dc >= 1 && dc < a.npos) ? w : 0.0f;
                pos_0 = a.wpos[0];
            }
        }

        // Block c into slot c % NS; blocks are issued PF ahead, also past the
        // last one (an empty buffer range: nothing is read), so that a wait
        // for at most (PF - 1) blocks' loads covers block c exactly.  Loads
        // return in issue order; the loop issues nothing else.
        auto issue = [&](int c) {
            unsigned char* sl = lds + (c % NS) * SLOT;
            const int row0 = 32 * (j0 + c);
            stage<D>(qb, row_stride, row0, q_end, row_bytes, sl, lo, false);
            stage<D>(qb, row_stride, row0, q_end, row_bytes, sl + C::ARR, lo, true);
            stage<D>(ob, row_stride, row0, q_end, row_bytes, sl + 2 * C::ARR, lo, false);
            stage<D>(ob, row_stride, row0, q_end, row_bytes, sl + 3 * C::ARR, lo, true);
            if constexpr (RAB) {
                // wave 0: the block's query timestamps; waves 1-3: wpos at
                // distances row0 - k0i - 128 + 64 (wv - 1) + lane
                unsigned char* ra = lds + NS * SLOT + (c % NS) * RABB_WORDS * 4;
                if (wv == 0)
                    load4_to_lds(make_rsrc32(a.ts + start + row0, min(q_end - row0, 32) * 4), ra,
                                 lane * 4);
                else
                    load4_to_lds(make_rsrc32(a.wpos, a.npos * 4),
                                 ra + 4 * RABB_TS + 256 * (wv - 1),
                                 4 * (row0 - k0i - 128 + 64 * (wv - 1) + lane));
            }
        };
#pragma unroll
        for (int c = 0; c < PF; ++c) issue(c);
        for (int c = 0; c < nblk; ++c) {
            __builtin_amdgcn_s_waitcnt(VMCNT_LE((PF - 1) * LT));
            __syncthreads();
            issue(c + PF);
            const unsigned char* sl = lds + (c % NS) * SLOT;
            const int q0 = 32 * (j0 + c);
            const bool skip = !live || q0 < kw0 || (TGT && kw0 >= hist && q0 > kw0);
            if (!skip) {
                f32x16 st = (f32x16){}, dp = (f32x16){};
                if constexpr (RAB) {
                    // rab / alpha for query q0 + 8(r/4) + 4g + r%4 and key kw0 + l32:
                    // distance q - key = window entry 128 - 32wv - l32 + 4g + 8(r/4) + r%4
                    const unsigned char* ra = lds + NS * SLOT + (c % NS) * RABB_WORDS * 4;
                    const float* win = reinterpret_cast<const float*>(ra + 4 * RABB_TS) +
                                       (128 - 32 * wv - l32 + 4 * g);
                    // position term of register r (candidate rows: see pos_c)
                    const bool cand = TGT && q0 + 31 >= hist;
                    auto posv = [&](int r) {
                        const float w = win[8 * (r >> 2) + (r & 3)];
                        if (!cand) return w;
                        const int qr = q0 + 8 * (r >> 2) + 4 * g + (r & 3);
                        return qr < hist ? w : (qr == kw0 + l32 ? pos_0 : pos_c);
                    };
                    // (query rows past the sequence read 0: a block holding
                    // them only looks nearer)
                    bool far = false;
                    if constexpr (D == 64)
                        far = rab_far(wave_min_i32(reinterpret_cast<const int*>(ra)[l32]), kmax,
                                      a.ntime);
                    if (far) {
                        const float tlast = ttab[0];
#pragma unroll
                        for (int r = 0; r < 16; ++r) st[r] = __builtin_fmaf(posv(r), a.bias_scale, tlast);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const u32x4 tq =
                                    *reinterpret_cast<const u32x4*>(ra + 4 * (4 * g + 8 * j));
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int f = ffbh_u32(tq[e] + c1);
                                st[4 * j + e] =
                                        __builtin_fmaf(posv(4 * j + e), a.bias_scale, ttab[f + 1]);
                            }
                        }
                    }
                }
                const RowReads<D> rr(lo);
#pragma unroll
                for (int ks = 0; ks < C::NKS; ++ks) {
                    st = M::mma(row_read<T, D>(sl, rr.r[ks]), kop[ks], st);
                    dp = M::mma(row_read<T, D>(sl + 2 * C::ARR, rr.r[ks]), vop[ks], dp);
                }
                // lane: key kw0 + l32; register r: query q0 + 8(r/4) + 4g + r%4
                const bool masked = q0 == kw0 || (TGT && kw0 + 31 >= hist);
                const int key = kw0 + l32;
                f32x16 p, ds;
                // A pair its query row does not see gets the score operand
                // +2^100: exp2 overflows to +inf, its reciprocal is 0, and the
                // pair's weight and dS come out as (signed) zeros.  The
                // selects sit under one uniform branch, so the pointwise pass
                // is one straight-line block for every block (a select folded
                // into it became a branch per element; two copies of it cost
                // registers).  With o = query - q0 - 4g (a constant per
                // register) and kq = key - q0 - 4g: the row sees the key iff
                // o >= kq and (key < hist or o == kq).
                if (masked) {
                    const int kq = key - q0 - 4 * g;
                    const bool kh = key < hist;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = 8 * (r >> 2) + (r & 3);
                        st[r] = (o >= kq && (kh || o == kq)) ? st[r] : 0x1p100f;
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr, dsr;
                    pointwise_m(st[r], dp[r], &pr, &dsr);
                    p[r] = pr;
                    ds[r] = dsr;
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x8 pf, df;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        pf[e] = p[8 * t + e];
                        df[e] = ds[8 * t + e];
                    }
                    const v8 pb = __builtin_convertvector(pf, v8);
                    const v8 db8 = __builtin_convertvector(df, v8);
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db) {
                        dv[db] = M::mma(tr_read<T, D>(sl + 3 * C::ARR, t, lo, db), pb, dv[db]);
                        dk[db] = M::mma(tr_read<T, D>(sl + C::ARR, t, lo, db), db8, dk[db]);
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(VMCNT_LE(0));
        __syncthreads();   // every read of the last block is done before the next item stages
        if (live) {
            const int64_t off = seq_base + (int64_t)kw0 * row_stride;
            store_rows<T, D>(a.dk + off, s - kw0, row_bytes, l32, g, dk, a.g_scale);
            // (the weights were m sig = silu(x) / -ln(2))
            store_rows<T, D>(a.dv + off, s - kw0, row_bytes, l32, g, dv, -BWD_LN2 * a.dv_scale);
        }
    }
}

// ---------------------------------------------------------------------------
// dQ.  Item (sequence, head, query tile): rows [128 qt, 128 qt + 128).  Wave
// wv owns rows wr0 .. wr0 + 31 and streams key blocks 0 .. up to its
// diagonal; with the target-aware mask, key blocks holding only candidates
// below the workgroup's rows are skipped altogether.  LDS slot: K (row reads),
// K (transposed), V (row reads).
// ---------------------------------------------------------------------------
// With the bias, the table gradients: a pair's score gradient (dS / n) goes
// to the position entry of its distance and to its time bucket.  (LDS float
// atomics cost on the order of a hundred cycles per instruction here, so the
// sums avoid them where they can.)
//  Position: a wave first sums its 32 x 32 block of dS along each diagonal
//  with DPP row shifts and lane swaps (lane l < 32 ends with the sum for
//  distance wr0 - k0 + l, lane 32 + l with wr0 - k0 + l - 32), then adds them
//  to a 256-entry ring of its own in LDS
//  (distance mod 256; plain read-add-write, the wave being its only writer).
//  A block of keys k0 .. k0+31 touches distances q0 - k0 - 31 .. q0 - k0 + 127
//  of the item's rows, so once block c is done, distances above
//  q0 - 32(c+1) + 127 are final for the item: the four rings' entries are
//  added to the workgroup's partial in global memory.
//  Time: each lane sums runs of equal (capped) buckets over its keys
//  (ascending, so with ordered timestamps a run usually spans the block, and
//  all pairs past the last bucket's gap share it) and adds a run to a
//  per-workgroup LDS bin when its bucket changes; runs in the last bucket,
//  nearly all of them past the diagonal blocks, stay in a register for the
//  whole launch and are summed over the wave once at its end (this measured
//  1.313 -> 1.249 ms for the bias backward at 16 x 4096; per-block wave sums
//  and LDS atomics before).  The bins go to the partial at the end.
//  Three workgroups per CU (168 VGPRs, no spills since the cross-lane sums
//  moved to DPP) for the bias forms at d = 64, whose waves then waited on LDS
//  for most of their cycles: 1.244 -> 1.126 ms for the causal form's backward at
//  16 x 4096; under the target-aware mask (about 30 spilled since the column
//  sums left LDS) 1.065 -> 0.921 ms at 16 x (3072 + 1024), where it had
//  measured slower with 70 spilled.  A spill reloaded inside the loop costs more than
//  its load: the compiler's wait for it counts the tile loads issued before
//  it too, so the next block's prefetch stops overlapping.
// Four workgroups per CU for the plain forms at d = 64 (128 VGPRs, no
// spills; 35 KB of LDS each): 0.577 -> 0.564 ms for the backward at
// 16 x 4096.
template <typename T, int D, bool FUSED, bool TGT, bool RAB = false>
__global__ __launch_bounds__(256, (!RAB && D == 64) ? 4 : (RAB && D == 64) ? 3 : 2)
void attn_bwd_dq(
        typename BwdArgsOf<RAB>::type a) {
    using C = BwdCfg<D>;
    using M = Mfma<T>;
    using v8 = typename M::v8;
    constexpr int SLOT = 3 * C::ARR;
    constexpr int PF = C::PF, NS = PF + 1;
    constexpr int LT = 3 * C::LPA;   // loads per wave per block
    constexpr int RAB_BYTES = RAB ? NS * RABB_WORDS * 4 : 0;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[NS * SLOT + RAB_BYTES];
    __shared__ int s_item[NQ];
    __shared__ LocalTables lt;
    __shared__ float ttab[RAB ? 33 : 1];   // time term by v_ffbh_u32(gap + 1) + 1, times -log2(e)
    __shared__ float ring[RAB ? 4 * 256 : 1];   // per wave: position-gradient sums by distance mod 256
    // time-gradient sums by bucket; [32]: candidates' pairs with themselves
    // (position distance 0, target-aware mask)
    __shared__ float tbins[RAB ? 33 : 1];
    static_assert(C::NW * 64 >= FUSE_SEQS && C::NW * 64 >= 32 * NQ, "fused tables need a thread per sequence");
    static_assert(!RAB || PF == 1, "bias: one block ahead");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = a.row_stride;
    const int row_bytes = (int)(row_stride * 2);
    const LaneOffsets<D> lo(lane, wv, row_bytes);
    float* gpart = nullptr;
    float tlast = 0.0f;   // this lane's time-gradient sum in the last bucket
    if constexpr (RAB) {
        if (tid < 33) ttab[tid] = a.wtime[rab_time_bucket(tid, a.ntime)] * a.bias_scale;
        if (tid < 33) tbins[tid] = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) ring[tid + 256 * i] = 0.0f;
        gpart = a.gpart + (int64_t)(blockIdx.x % a.nparts) * a.gstride;
    }
    // Adds the four rings' entries of distances [lo_d, hi_d] (at most 256 of
    // them) to the partial and clears them; called by every thread between
    // barriers.
    auto flush_ring = [&](int lo_d, int hi_d) {
        if constexpr (RAB) {
            const int dd = hi_d - tid;
            if (dd >= lo_d && dd >= 0) {
                const int e = dd & 255;
                const float x = ring[e] + ring[256 + e] + ring[512 + e] + ring[768 + e];
                ring[e] = ring[256 + e] = ring[512 + e] = ring[768 + e] = 0.0f;
                if (dd < a.npos && x != 0.0f)
                    __hip_atomic_fetch_add(gpart + dd, x * a.dv_scale, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };

    Tables tb;
    if constexpr (FUSED)
        tb = build_local_tables(lt, reinterpret_cast<int*>(lds), a.offsets, a.num_seqs, H, C::ROWS,
                                a.wl.ctl);
    else
        tb = global_tables(a.wl);
    clear_sets(a.wl.ctl, a.wl.set + 2, 1);   // (the next call's sets: see the launcher)
    ItemSource src(a.wl.ctl, a.wl.set);
    int qx, w;
    while (src.next(tb, s_item, &qx, &w)) {
        const Item it = decode_item(tb, a.num_seqs, H, qx, w);
        const int seq = __builtin_amdgcn_readfirstlane(it.seq);
        const int head = __builtin_amdgcn_readfirstlane(it.head);
        const int qtile = __builtin_amdgcn_readfirstlane(it.qtile);
        const int start = __builtin_amdgcn_readfirstlane(a.offsets[seq]);
        const int s = __builtin_amdgcn_readfirstlane(a.offsets[seq + 1]) - start;
        int hist = s;
        if constexpr (TGT) hist = s - min(max(__builtin_amdgcn_readfirstlane(a.ntgt[seq]), 0), s);
        const int q0 = qtile * C::ROWS;
        const int wr0 = q0 + 32 * wv;
        const bool live = wr0 < s;
        const int kv_end = min(s, q0 + C::ROWS);
        // Key blocks 0 .. nh-1 hold history keys; blocks nh .. q0/32 - 1 hold
        // only candidates below every row of the item and are jumped over.
        const int nb_all = (kv_end + 31) / 32;
        const int nh = TGT ? (hist + 31) / 32 : nb_all;
        const int jump = TGT ? max(q0 / 32 - nh, 0) : 0;
        const int nblk = nb_all - jump;
        auto k0_of = [&](int c) { return 32 * (c >= nh ? c + jump : c); };
        // The bias sees a candidate row (row >= hist) at position hist: the
        // item's distances are those of effective rows min(row, hist), which
        // start at q0e.
        const int q0e = TGT ? min(q0, hist) : q0;
        const bool cand_w = TGT && wr0 + 31 >= hist;   // the wave has candidate rows
        const int64_t seq_base = (int64_t)start * H * D + (int64_t)head * a.head_stride;
        const uint16_t* kb = a.k + seq_base;
        const uint16_t* vb = a.v + seq_base;

        v8 qop[C::NKS], oop[C::NKS];
        load_rows_b<T, D>(a.q + seq_base + (int64_t)wr0 * row_stride, row_stride, s - wr0,
                          row_bytes, l32, g, qop);
        load_rows_b<T, D>(a.dout + seq_base + (int64_t)wr0 * row_stride, row_stride, s - wr0,
                          row_bytes, l32, g, oop);
        // Q * (-alpha log2(e)), rounded to T, as K in the dK/dV kernel.
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks)
            qop[ks] = __builtin_convertvector(
                    __builtin_convertvector(qop[ks], f32x8) * a.score_scale, v8);
        f32x16 dq[C::NDB];
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) dq[db] = (f32x16){};
        // With the bias: ts of this lane's query + 1.
        uint32_t trp1 = 0;
        int rmin = 0;   // the wave's earliest query timestamp
        float pos_0 = 0.0f, d0 = 0.0f;   // wpos[0]; this lane's candidate-with-itself dS
        if constexpr (RAB && TGT) pos_0 = a.wpos[0];
        if constexpr (RAB) {
            trp1 = __builtin_amdgcn_raw_buffer_load_b32(
                           make_rsrc(a.ts + start + wr0, (int64_t)(s - wr0) * 4), l32 * 4, 0, 0) +
                   1u;
            if constexpr (D == 64)
                rmin = wave_min_i32(wr0 + l32 < s ? (int)(trp1 - 1u) : INT32_MAX);
        }

        // (staged PF ahead as in the dK/dV kernel)
        auto issue = [&](int c) {
            unsigned char* sl = lds + (c % NS) * SLOT;
            const int row0 = 32 * (c >= nh ? c + jump : c);
            stage<D>(kb, row_stride, row0, kv_end, row_bytes, sl, lo, false);
            stage<D>(kb, row_stride, row0, kv_end, row_bytes, sl + C::ARR, lo, true);
            stage<D>(vb, row_stride, row0, kv_end, row_bytes, sl + 2 * C::ARR, lo, false);
            if constexpr (RAB) {
                // wave 0: the block's key timestamps; waves 1-3: wpos at
                // distances q0e - row0 - 32 + 64 (wv - 1) + lane
                unsigned char* ra = lds + NS * SLOT + (c % NS) * RABB_WORDS * 4;
                if (wv == 0)
                    load4_to_lds(make_rsrc32(a.ts + start + row0, min(kv_end - row0, 32) * 4), ra,
                                 lane * 4);
                else
                    load4_to_lds(make_rsrc32(a.wpos, a.npos * 4),
                                 ra + 4 * RABB_TS + 256 * (wv - 1),
                                 4 * (q0e - row0 - 32 + 64 * (wv - 1) + lane));
            }
        };
#pragma unroll
        for (int c = 0; c < PF; ++c) issue(c);
        for (int c = 0; c < nblk; ++c) {
            __builtin_amdgcn_s_waitcnt(VMCNT_LE((PF - 1) * LT));
            __syncthreads();
            issue(c + PF);
            // (block c-1 done by every wave: distances only it or the blocks
            // jumped over could touch are final; what can still be non-zero
            // lies within block c-1's own range)
            if (c > 0)
                flush_ring(max(q0e + 128 - k0_of(c), q0e - k0_of(c - 1) - 31),
                           q0e + 127 - k0_of(c - 1));
            const unsigned char* sl = lds + (c % NS) * SLOT;
            const int k0 = 32 * (c >= nh ? c + jump : c);
            const bool skip = !live || k0 > wr0 || (TGT && k0 >= hist && k0 + 31 < wr0);
            if (!skip) {
                f32x16 st = (f32x16){}, dp = (f32x16){};
                u32x4 tk[4];
                bool far = false;
                if constexpr (RAB) {
                    // rab / alpha for query wr0 + l32 and key k0 + 8(r/4) + 4g + r%4:
                    // distance = window entry erow - q0e + 32 - 4g - 8(r/4) - r%4,
                    // erow the lane's effective row (a candidate and its own
                    // key: distance 0, pos_0)
                    const unsigned char* ra = lds + NS * SLOT + (c % NS) * RABB_WORDS * 4;
                    const int erow = TGT ? min(wr0 + l32, hist) : wr0 + l32;
                    const float* win = reinterpret_cast<const float*>(ra + 4 * RABB_TS) +
                                       (erow - q0e + 5 - 4 * g);
                    auto posv = [&](int r) {
                        const float w = win[27 - 8 * (r >> 2) - (r & 3)];
                        if (!cand_w) return w;
                        const int key = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
                        return (wr0 + l32 >= hist && key == wr0 + l32) ? pos_0 : w;
                    };
                    // (keys past the sequence read 0: a block holding them
                    // only looks nearer)
                    if constexpr (D == 64)
                        far = rab_far(rmin,
                                      wave_max_i32(reinterpret_cast<const int*>(ra)[l32]),
                                      a.ntime);
                    if (far) {
                        const float tlast = ttab[0];
#pragma unroll
                        for (int r = 0; r < 16; ++r) st[r] = __builtin_fmaf(posv(r), a.bias_scale, tlast);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            tk[j] = *reinterpret_cast<const u32x4*>(ra + 4 * (4 * g + 8 * j));
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int f = ffbh_u32(trp1 - tk[j][e]);
                                st[4 * j + e] =
                                        __builtin_fmaf(posv(4 * j + e), a.bias_scale, ttab[f + 1]);
                            }
                        }
                    }
                }
                const RowReads<D> rr(lo);
#pragma unroll
                for (int ks = 0; ks < C::NKS; ++ks) {
                    st = M::mma(row_read<T, D>(sl, rr.r[ks]), qop[ks], st);
                    dp = M::mma(row_read<T, D>(sl + 2 * C::ARR, rr.r[ks]), oop[ks], dp);
                }
                // lane: query wr0 + l32; register r: key k0 + 8(r/4) + 4g + r%4
                const bool masked = k0 + 31 >= wr0 || (TGT && k0 + 31 >= hist);
                const int row = wr0 + l32;
                f32x16 ds;
                // A pair the row does not see gets the score operand +2^100:
                // exp2 overflows to +inf, its reciprocal is 0, so the pair's
                // weight and dS come out as (signed) zeros with no select
                // after the pointwise pass.  The selects sit under one
                // uniform branch, so the pointwise pass stays one
                // straight-line block (a select per element folded into it
                // became a branch per element, with the loop-invariant key
                // offsets spilled to scratch).  With o = key - k0 - 4g (a
                // constant per register): the row sees o <= eq and (o < hh
                // or o == eq).
                if (masked) {
                    const int eq = row - k0 - 4 * g;
                    const int hh = hist - k0 - 4 * g;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = 8 * (r >> 2) + (r & 3);
                        st[r] = (o <= eq && (o < hh || o == eq)) ? st[r] : 0x1p100f;
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr, dsr;
                    pointwise_m(st[r], dp[r], &pr, &dsr);
                    ds[r] = dsr;
                }
                if constexpr (RAB) {
                    f32x16 dgl = ds;   // the pairs credited along diagonals (row - key)
                    if constexpr (TGT) {
                        if (cand_w) {
                            // A candidate row's pairs with history keys go to
                            // distance hist - key (column sums over the wave's
                            // candidate rows), its pair with itself to
                            // distance 0 (d0, added once per item).
                            const bool crow = row >= hist;
                            f32x16 dcol;
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int key = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
                                dcol[r] = (crow && key < hist) ? ds[r] : 0.0f;
                                d0 += (crow && key == row) ? ds[r] : 0.0f;
                                dgl[r] = crow ? 0.0f : ds[r];
                            }
                            const float u = half_wave_column_sum(dcol, l32);
                            const int cr = (l32 >> 1) & 15;
                            const int ckey = k0 + 8 * (cr >> 2) + 4 * g + (cr & 3);
                            if ((l32 & 1) == 0 && ckey < hist)
                                ring[256 * wv + ((hist - ckey) & 255)] += u;
                        }
                    }
                    // distance of register r: wr0 + l32 - k0 - 4g - (8(r/4) + r%4);
                    // masked pairs add exactly zero
                    // Diagonal sums: register r of lane (g, l) holds query wr0 + l,
                    // key k0 + o, o = 8(r/4) + 4g + r%4.  Lane (g, l) gathers
                    // register r of lane (g, (l + S) mod 32), S = o - 4g (see
                    // diag_step): a pair of distance l - 4g, or, when l + S
                    // wraps past 31, of distance l - 4g - 32 (relative to
                    // wr0 - k0).  Every pair is taken by exactly one lane.  (A
                    // wave of candidate rows only has nothing to add along
                    // diagonals: skipped.)
                    if (!TGT || wr0 < hist) {
                        float dhi = 0.0f, dlo = 0.0f;
                        diag_steps(dgl, dhi, dlo, std::make_integer_sequence<int, 16>{});
                        // The halves combined: one v_permlane32_swap (the upper
                        // 32 lanes of dhi trade places with the lower 32 of dlo)
                        // leaves the first half's dhi, dlo in lanes 0-31, 32-63
                        // of s0 and the second half's in s1; the second half's
                        // sums sit 4 distances lower, so s1 is read 4 lanes on
                        // (mod 64, which carries its dhi of distances -4 .. -1
                        // into the wrapped sums).  Lanes 0-31 end with distance
                        // l, lanes 32-63 with l - 32, and every lane adds its
                        // sum to the ring at its own distance.
                        const unsigned hi_u = __builtin_bit_cast(unsigned, dhi);
                        const unsigned lo_u = __builtin_bit_cast(unsigned, dlo);
                        const auto sw = __builtin_amdgcn_permlane32_swap(hi_u, lo_u, false, false);
                        const unsigned s0 = sw[0], s1 = sw[1];
                        const float s1n = __shfl(__builtin_bit_cast(float, s1), (lane + 4) & 63, 64);
                        float* rw = ring + 256 * wv;
                        rw[(wr0 - k0 + l32 - 32 * g) & 255] += __builtin_bit_cast(float, s0) + s1n;
                    }
                    // Time buckets: runs of equal buckets along the lane's keys.  The
                    // capped bucket of v_ffbh_u32 result f is min(31 - f, ntime - 1)
                    // (f = -1, a gap of -1, gives 32: the last bucket too).
                    const int cap = a.ntime - 1;
                    int prev = cap;
                    float run = 0.0f;
                    if (D == 64 && far) {   // every pair in the last bucket
#pragma unroll
                        for (int r = 0; r < 16; ++r) run += ds[r];
                    } else {
                        // (the keys' timestamps read again: kept in registers
                        // across the products they pushed this kernel's
                        // loop-invariant values out to scratch)
                        // (the empty asm with a memory clobber keeps the
                        // compiler from reusing the first read)
                        const unsigned char* ra = lds + NS * SLOT + (c % NS) * RABB_WORDS * 4;
                        asm volatile("" ::: "memory");
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            tk[j] = *reinterpret_cast<const u32x4*>(ra + 4 * (4 * g + 8 * j));
                        prev = min(31 - ffbh_u32(trp1 - tk[0][0]), cap);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int b = min(31 - ffbh_u32(trp1 - tk[r >> 2][r & 3]), cap);
                            if (b != prev) {
                                atomicAdd(&tbins[prev], run);
                                run = 0.0f;
                                prev = b;
                            }
                            run += ds[r];
                        }
                    }
                    // (the last bucket, where nearly every run ends: in a register)
                    if (prev == cap)
                        tlast += run;
                    else
                        atomicAdd(&tbins[prev], run);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x8 df;
#pragma unroll
                    for (int e = 0; e < 8; ++e) df[e] = ds[8 * t + e];
                    const v8 db8 = __builtin_convertvector(df, v8);
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db)
                        dq[db] = M::mma(tr_read<T, D>(sl + C::ARR, t, lo, db), db8, dq[db]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(VMCNT_LE(0));
        __syncthreads();
        if (live)
            store_rows<T, D>(a.dq + seq_base + (int64_t)wr0 * row_stride, s - wr0, row_bytes, l32,
                             g, dq, a.g_scale);
        if constexpr (RAB) {
            // the item's remaining distances: those of its last block
            // (every ring update of the item is done: the barrier above)
            const int last = q0e - k0_of(nblk - 1);
            flush_ring(last - 31, last + 127);
            if (cand_w) {
                float t = d0;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
                if (lane == 0 && t != 0.0f) atomicAdd(&tbins[32], t);
            }
        }
    }
    if constexpr (RAB) {
        float t = tlast;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, 64);
        if (lane == 0 && t != 0.0f) atomicAdd(&tbins[a.ntime - 1], t);
        __syncthreads();
        if (tid < a.ntime && tbins[tid] != 0.0f)
            __hip_atomic_fetch_add(gpart + a.npos + tid, tbins[tid] * a.dv_scale,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (TGT && tid == 32 && tbins[32] != 0.0f)
            __hip_atomic_fetch_add(gpart, tbins[32] * a.dv_scale, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <typename T, int D, bool TGT>
hipError_t launch_bwd_typed(const BwdParams& p, WorkList wl, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop) {
    BwdArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.dout = static_cast<const uint16_t*>(p.dout);
    a.dq = static_cast<uint16_t*>(p.dq);
    a.dk = static_cast<uint16_t*>(p.dk);
    a.dv = static_cast<uint16_t*>(p.dv);
    a.offsets = p.offsets;
    a.ntgt = p.num_targets;
    a.num_seqs = p.num_seqs;
    a.heads = p.heads;
    a.row_stride = p.dense ? p.d : (int64_t)p.heads * p.d;
    a.head_stride = p.dense ? p.dense_len * p.d : p.d;
    a.score_scale = -p.alpha * BWD_LOG2E;
    a.dv_scale = 1.0f / p.n;
    a.g_scale = p.alpha / p.n;
    using Fn = void (*)(BwdArgs);
    const Fn f_dkv = wl.fused ? attn_bwd_dkv<T, D, true, TGT> : attn_bwd_dkv<T, D, false, TGT>;
    const Fn f_dq = wl.fused ? attn_bwd_dq<T, D, true, TGT> : attn_bwd_dq<T, D, false, TGT>;
    static int grids[2][2] = {};
    int& g_dkv = grids[wl.fused ? 1 : 0][0];
    int& g_dq = grids[wl.fused ? 1 : 0][1];
    if (!g_dkv) g_dkv = resident_grid(f_dkv, 256);
    if (!g_dq) g_dq = resident_grid(f_dq, 256);
    // dK/dV on this call's first counter set, dQ on the next; each launch
    // clears the set two after its own, so the two clear the next call's pair.
    a.wl = wl;
    if (start)
        hipExtLaunchKernelGGL(f_dkv, dim3(g_dkv), dim3(256), 0, stream, start, nullptr, 0, a);
    else
        hipLaunchKernelGGL(f_dkv, dim3(g_dkv), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.wl.set = (wl.set + 1) % NSETS;
    if (stop)
        hipExtLaunchKernelGGL(f_dq, dim3(g_dq), dim3(256), 0, stream, nullptr, stop, 0, a);
    else
        hipLaunchKernelGGL(f_dq, dim3(g_dq), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Bias gradients: the partials are zeroed first and summed last.
__global__ void rab_zero_kernel(float* p, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

__global__ void rab_reduce_kernel(const float* gpart, int nparts, int gstride, int npos,
                                  int ntime, float* dpos, float* dtime) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= npos + ntime) return;
    float acc = 0.0f;   // (position entries, then time buckets at npos + b)
    for (int w = 0; w < nparts; ++w) acc += gpart[(int64_t)w * gstride + j];
    if (j < npos)
        dpos[j] = acc;
    else
        dtime[j - npos] = acc;
}

template <typename T, int D, bool TGT>
hipError_t launch_bwd_rab(const BwdParams& p, WorkList wl, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
    BwdArgsRab a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.dout = static_cast<const uint16_t*>(p.dout);
    a.dq = static_cast<uint16_t*>(p.dq);
    a.dk = static_cast<uint16_t*>(p.dk);
    a.dv = static_cast<uint16_t*>(p.dv);
    a.offsets = p.offsets;
    a.ntgt = TGT ? p.num_targets : nullptr;
    a.num_seqs = p.num_seqs;
    a.heads = p.heads;
    a.row_stride = (int64_t)p.heads * p.d;
    a.head_stride = p.d;
    a.score_scale = -p.alpha * BWD_LOG2E;
    a.dv_scale = 1.0f / p.n;
    a.g_scale = p.alpha / p.n;
    a.ts = p.timestamps;
    a.wpos = p.pos_bias;
    a.wtime = p.time_bias;
    a.gpart = p.rab_partials;
    a.npos = p.num_pos;
    a.ntime = p.num_time;
    a.gstride = rab_partial_stride(p.num_pos);
    a.nparts = RAB_PARTS;
    a.bias_scale = -BWD_LOG2E;
    using Fn = void (*)(BwdArgsRab);
    const Fn f_dkv = wl.fused ? attn_bwd_dkv<T, D, true, TGT, true>
                              : attn_bwd_dkv<T, D, false, TGT, true>;
    const Fn f_dq = wl.fused ? attn_bwd_dq<T, D, true, TGT, true>
                             : attn_bwd_dq<T, D, false, TGT, true>;
    static int grids[2][2] = {};
    int& g_dkv = grids[wl.fused ? 1 : 0][0];
    int& g_dq = grids[wl.fused ? 1 : 0][1];
    if (!g_dkv) g_dkv = resident_grid(f_dkv, 256);
    if (!g_dq) g_dq = resident_grid(f_dq, 256);
    const int64_t cells = (int64_t)RAB_PARTS * a.gstride;
    hipLaunchKernelGGL(rab_zero_kernel, dim3(256), dim3(256), 0, stream, a.gpart, cells);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.wl = wl;
    if (start)
        hipExtLaunchKernelGGL(f_dkv, dim3(g_dkv), dim3(256), 0, stream, start, nullptr, 0, a);
    else
        hipLaunchKernelGGL(f_dkv, dim3(g_dkv), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.wl.set = (wl.set + 1) % NSETS;
    hipLaunchKernelGGL(f_dq, dim3(g_dq), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_out = p.num_pos + p.num_time;
    if (stop)
        hipExtLaunchKernelGGL(rab_reduce_kernel, dim3((n_out + 255) / 256), dim3(256), 0, stream,
                              nullptr, stop, 0, (const float*)a.gpart, a.nparts, a.gstride,
                              p.num_pos, p.num_time, p.d_pos_bias, p.d_time_bias);
    else
        hipLaunchKernelGGL(rab_reduce_kernel, dim3((n_out + 255) / 256), dim3(256), 0, stream,
                           (const float*)a.gpart, a.nparts, a.gstride, p.num_pos, p.num_time,
                           p.d_pos_bias, p.d_time_bias);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_mask(const BwdParams& p, WorkList wl, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
    if (p.timestamps)
        return p.num_targets ? launch_bwd_rab<T, D, true>(p, wl, stream, start, stop)
                             : launch_bwd_rab<T, D, false>(p, wl, stream, start, stop);
    return p.num_targets ? launch_bwd_typed<T, D, true>(p, wl, stream, start, stop)
                         : launch_bwd_typed<T, D, false>(p, wl, stream, start, stop);
}

// ---------------------------------------------------------------------------
// fp32: v_mfma_f32_32x32x2_f32, same two kernels and item shapes, tiles staged
// synchronously into padded LDS arrays (like the fp32 forward).  A lane's
// k-slice is one element: accumulator register r of lane (l32, g) holds row
// 8(r/4) + 4g + r%4, which is exactly the k index of k-step r of a product
// that contracts over those rows, so P, dS and dS^T feed the second products
// register by register.
// ---------------------------------------------------------------------------
struct BwdArgsF32 {
    const float* q;
    const float* k;
    const float* v;
    const float* dout;
    float* dq;
    float* dk;
    float* dv;
    const int32_t* offsets;
    const int32_t* ntgt;
    WorkList wl;
    int64_t row_stride;
    int64_t head_stride;
    int num_seqs;
    int heads;
    float alpha;
    float dv_scale;
    float g_scale;
    // relative attention bias (RAB instantiations only)
    const int32_t* ts;
    const float* wpos;
    const float* wtime;
    float* gpart;   // [nparts][gstride]: npos position entries, then the time buckets
    int npos;
    int ntime;
    int gstride;
    int nparts;
    float bias_scale;   // 1 / alpha
};

// The bias of pair (row, key) of a sequence over alpha, read from global
// memory (the float32 kernels are the reference-precision path, not the fast
// one); ttab is the time table by v_ffbh_u32(gap + 1) + 1, already over
// alpha.  Rows or keys at or past the sequence's end get 0 (their terms are
// zero anyway).  *dist and *bucket name the table entries the pair uses; a
// candidate row (row >= hist) sits right after the history: distance
// hist - key to a history key, 0 to itself.
__device__ __forceinline__ float bias_over_alpha_f32(const BwdArgsF32& a, const float* ttab,
                                                     int start, int s, int hist, int row, int key,
                                                     int* dist, int* bucket) {
    *dist = row >= hist ? (key == row ? 0 : hist - key) : row - key;
    *bucket = 0;
    if (row >= s || key >= s) return 0.0f;
    const uint32_t x = (uint32_t)a.ts[start + row] + 1u - (uint32_t)a.ts[start + key];
    const int f = ffbh_u32(x);
    *bucket = rab_time_bucket(f + 1, a.ntime);
    const float pos = (*dist >= 0 && *dist < a.npos) ? a.wpos[*dist] * a.bias_scale : 0.0f;
    return pos + ttab[f + 1];
}

template <int D>
struct BwdCfgF32 {
    static constexpr int NW = 4;
    static constexpr int ROWS = 32 * NW;
    static constexpr int STR = D + 2;                    // floats per LDS row
    static constexpr int CHUNKS = 32 * D / 4 / (NW * 64);   // float4 loads per thread per array
    static_assert(CHUNKS * NW * 64 * 4 == 32 * D, "array must split evenly");
};

// Rows [row0, row0 + 32) of one tensor into a padded LDS array; rows at or
// past rows_avail as zero.  Every thread of the workgroup takes part.
template <int D>
__device__ __forceinline__ void stage_f32(const float* base, int64_t row_stride, int row0,
                                          int rows_avail, float* arr) {
    using C = BwdCfgF32<D>;
#pragma unroll
    for (int i = 0; i < C::CHUNKS; ++i) {
        const int id = threadIdx.x + i * C::NW * 64;
        const int r = id / (D / 4), c4 = id % (D / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row0 + r < rows_avail)
            x = *reinterpret_cast<const float4*>(base + (int64_t)(row0 + r) * row_stride + 4 * c4);
        float* d = arr + r * C::STR + 4 * c4;
        d[0] = x.x;
        d[1] = x.y;
        d[2] = x.z;
        d[3] = x.w;
    }
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool FUSED, bool TGT, bool RAB = false>
__global__ __launch_bounds__(256) void attn_bwd_dkv_f32(BwdArgsF32 a) {
    using C = BwdCfgF32<D>;
    constexpr int NDB = D / 32;
    __shared__ __attribute__((aligned(16))) float ql[32 * C::STR];
    __shared__ __attribute__((aligned(16))) float ol[32 * C::STR];
    __shared__ int s_item[NQ];
    __shared__ LocalTables lt;
    __shared__ int tbl_scratch[FUSE_SEQS];
    __shared__ float ttab[RAB ? 33 : 1];
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = a.row_stride;
    if constexpr (RAB) {
        if (threadIdx.x < 33)
            ttab[threadIdx.x] = a.wtime[rab_time_bucket(threadIdx.x, a.ntime)] * a.bias_scale;
    }

    Tables tb;
    if constexpr (FUSED)
        tb = build_local_tables(lt, tbl_scratch, a.offsets, a.num_seqs, H, C::ROWS, a.wl.ctl);
    else
        tb = global_tables(a.wl);
    clear_sets(a.wl.ctl, a.wl.set + 2, 1);   // (the next call's sets: see the launcher)
    ItemSource src(a.wl.ctl, a.wl.set);
    int qx, w;
    while (src.next(tb, s_item, &qx, &w)) {
        const Item it = decode_item(tb, a.num_seqs, H, qx, w);
        const int start = a.offsets[it.seq];
        const int s = a.offsets[it.seq + 1] - start;
        const int ntile = (s + C::ROWS - 1) / C::ROWS;
        const int kt = ntile - 1 - it.qtile;
        const int hist = TGT ? s - min(max(a.ntgt[it.seq], 0), s) : s;
        const int k0i = kt * C::ROWS;
        const int kw0 = k0i + 32 * wv;
        const bool live = kw0 < s;
        const int q_end = (TGT && k0i >= hist) ? min(s, k0i + C::ROWS) : s;
        const int j0 = k0i / 32;
        const int nblk = (q_end + 31) / 32 - j0;
        const int64_t seq_base = (int64_t)start * H * D + (int64_t)it.head * a.head_stride;
        const int key = kw0 + l32;
        // B operands: K and V of the lane's key, head-dim element 2 ks + g.
        float kop[D / 2], vop[D / 2];
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks) {
            const bool ok = key < s;
            kop[ks] = ok ? a.k[seq_base + (int64_t)key * row_stride + 2 * ks + g] : 0.0f;
            vop[ks] = ok ? a.v[seq_base + (int64_t)key * row_stride + 2 * ks + g] : 0.0f;
        }
        f32x16 dk[NDB], dv[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = (f32x16){};

        for (int c = 0; c < nblk; ++c) {
            const int q0 = 32 * (j0 + c);
            stage_f32<D>(a.q + seq_base, row_stride, q0, q_end, ql);
            stage_f32<D>(a.dout + seq_base, row_stride, q0, q_end, ol);
            __syncthreads();
            const bool skip = !live || q0 < kw0 || (TGT && kw0 >= hist && q0 > kw0);
            if (!skip) {
                f32x16 st = (f32x16){}, dp = (f32x16){};
#pragma unroll
                for (int ks = 0; ks < D / 2; ++ks) {
                    st = mfma_f32(ql[l32 * C::STR + 2 * ks + g], kop[ks], st);
                    dp = mfma_f32(ol[l32 * C::STR + 2 * ks + g], vop[ks], dp);
                }
                const bool masked = q0 == kw0 || (TGT && kw0 + 31 >= hist);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr, dsr;
                    const int qrow = 8 * (r >> 2) + 4 * g + (r & 3);   // row inside the block
                    if constexpr (RAB) {
                        int dist, bucket;
                        st[r] += bias_over_alpha_f32(a, ttab, start, s, hist, q0 + qrow, key,
                                                     &dist, &bucket);
                    }
                    pointwise(st[r], dp[r], a.alpha, &pr, &dsr);
                    if (masked) {
                        const int qr = q0 + qrow;
                        const bool keep = key <= qr && (key < hist || key == qr);
                        pr = keep ? pr : 0.0f;
                        dsr = keep ? dsr : 0.0f;
                    }
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        dv[db] = mfma_f32(ol[qrow * C::STR + 32 * db + l32], pr, dv[db]);
                        dk[db] = mfma_f32(ql[qrow * C::STR + 32 * db + l32], dsr, dk[db]);
                    }
                }
            }
            __syncthreads();
        }
        if (live) {
            // lane: key; registers: head-dim rows 32 db + 8 (r/4) + 4 g + r%4
            if (key < s) {
                float* pk = a.dk + seq_base + (int64_t)key * row_stride;
                float* pv = a.dv + seq_base + (int64_t)key * row_stride;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int e = 32 * db + 8 * i + 4 * g;
                        *reinterpret_cast<float4*>(pk + e) =
                                make_float4(dk[db][4 * i] * a.g_scale, dk[db][4 * i + 1] * a.g_scale,
                                            dk[db][4 * i + 2] * a.g_scale, dk[db][4 * i + 3] * a.g_scale);
                        *reinterpret_cast<float4*>(pv + e) =
                                make_float4(dv[db][4 * i] * a.dv_scale, dv[db][4 * i + 1] * a.dv_scale,
                                            dv[db][4 * i + 2] * a.dv_scale,
                                            dv[db][4 * i + 3] * a.dv_scale);
                    }
            }
        }
    }
}

template <int D, bool FUSED, bool TGT, bool RAB = false>
__global__ __launch_bounds__(256) void attn_bwd_dq_f32(BwdArgsF32 a) {
    using C = BwdCfgF32<D>;
    constexpr int NDB = D / 32;
    __shared__ __attribute__((aligned(16))) float kl[32 * C::STR];
    __shared__ __attribute__((aligned(16))) float vl[32 * C::STR];
    __shared__ int s_item[NQ];
    __shared__ LocalTables lt;
    __shared__ int tbl_scratch[FUSE_SEQS];
    __shared__ float ttab[RAB ? 33 : 1];
    __shared__ float tbins[RAB ? 32 : 1];   // time-gradient sums by bucket
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = a.row_stride;
    // Table gradients: position entries straight into this workgroup's
    // partial with float atomics, time buckets summed in LDS and added to the
    // partial at the end.
    float* gpart = nullptr;
    if constexpr (RAB) {
        if (threadIdx.x < 33)
            ttab[threadIdx.x] = a.wtime[rab_time_bucket(threadIdx.x, a.ntime)] * a.bias_scale;
        if (threadIdx.x < 32) tbins[threadIdx.x] = 0.0f;
        gpart = a.gpart + (int64_t)(blockIdx.x % a.nparts) * a.gstride;
    }

    Tables tb;
    if constexpr (FUSED)
        tb = build_local_tables(lt, tbl_scratch, a.offsets, a.num_seqs, H, C::ROWS, a.wl.ctl);
    else
        tb = global_tables(a.wl);
    clear_sets(a.wl.ctl, a.wl.set + 2, 1);   // (the next call's sets: see the launcher)
    ItemSource src(a.wl.ctl, a.wl.set);
    int qx, w;
    while (src.next(tb, s_item, &qx, &w)) {
        const Item it = decode_item(tb, a.num_seqs, H, qx, w);
        const int start = a.offsets[it.seq];
        const int s = a.offsets[it.seq + 1] - start;
        const int hist = TGT ? s - min(max(a.ntgt[it.seq], 0), s) : s;
        const int q0 = it.qtile * C::ROWS;
        const int wr0 = q0 + 32 * wv;
        const bool live = wr0 < s;
        const int kv_end = min(s, q0 + C::ROWS);
        const int nb_all = (kv_end + 31) / 32;
        const int nh = TGT ? (hist + 31) / 32 : nb_all;
        const int jump = TGT ? max(q0 / 32 - nh, 0) : 0;
        const int nblk = nb_all - jump;
        const int64_t seq_base = (int64_t)start * H * D + (int64_t)it.head * a.head_stride;
        const int row = wr0 + l32;
        float qop[D / 2], oop[D / 2];
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks) {
            const bool ok = row < s;
            qop[ks] = ok ? a.q[seq_base + (int64_t)row * row_stride + 2 * ks + g] : 0.0f;
            oop[ks] = ok ? a.dout[seq_base + (int64_t)row * row_stride + 2 * ks + g] : 0.0f;
        }
        f32x16 dq[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db] = (f32x16){};

        for (int c = 0; c < nblk; ++c) {
            const int k0 = 32 * (c >= nh ? c + jump : c);
            stage_f32<D>(a.k + seq_base, row_stride, k0, kv_end, kl);
            stage_f32<D>(a.v + seq_base, row_stride, k0, kv_end, vl);
            __syncthreads();
            const bool skip = !live || k0 > wr0 || (TGT && k0 >= hist && k0 + 31 < wr0);
            if (!skip) {
                f32x16 st = (f32x16){}, dp = (f32x16){};
#pragma unroll
                for (int ks = 0; ks < D / 2; ++ks) {
                    st = mfma_f32(kl[l32 * C::STR + 2 * ks + g], qop[ks], st);
                    dp = mfma_f32(vl[l32 * C::STR + 2 * ks + g], oop[ks], dp);
                }
                const bool masked = k0 + 31 >= wr0 || (TGT && k0 + 31 >= hist);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr, dsr;
                    const int krow = 8 * (r >> 2) + 4 * g + (r & 3);   // key inside the block
                    int dist = 0, bucket = 0;
                    if constexpr (RAB)
                        st[r] += bias_over_alpha_f32(a, ttab, start, s, hist, row, k0 + krow,
                                                     &dist, &bucket);
                    pointwise(st[r], dp[r], a.alpha, &pr, &dsr);
                    if (masked) {
                        const int kk = k0 + krow;
                        dsr = (kk <= row && (kk < hist || kk == row)) ? dsr : 0.0f;
                    }
                    if constexpr (RAB) {
                        // (pairs past the sequence or the diagonal have dsr = 0)
                        if (dsr != 0.0f) {
                            if (dist < a.npos)
                                __hip_atomic_fetch_add(gpart + dist, dsr * a.dv_scale,
                                                       __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                            atomicAdd(&tbins[bucket], dsr);
                        }
                    }
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        dq[db] = mfma_f32(kl[krow * C::STR + 32 * db + l32], dsr, dq[db]);
                }
            }
            __syncthreads();
        }
        if (live && row < s) {
            float* pq = a.dq + seq_base + (int64_t)row * row_stride;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 32 * db + 8 * i + 4 * g;
                    *reinterpret_cast<float4*>(pq + e) =
                            make_float4(dq[db][4 * i] * a.g_scale, dq[db][4 * i + 1] * a.g_scale,
                                        dq[db][4 * i + 2] * a.g_scale, dq[db][4 * i + 3] * a.g_scale);
                }
        }
    }
    if constexpr (RAB) {
        __syncthreads();
        if (threadIdx.x < a.ntime && tbins[threadIdx.x] != 0.0f)
            __hip_atomic_fetch_add(gpart + a.npos + threadIdx.x, tbins[threadIdx.x] * a.dv_scale,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int D, bool TGT, bool RAB = false>
hipError_t launch_bwd_f32_typed(const BwdParams& p, WorkList wl, hipStream_t stream,
                                hipEvent_t start, hipEvent_t stop) {
    BwdArgsF32 a;
    a.q = static_cast<const float*>(p.q);
    a.k = static_cast<const float*>(p.k);
    a.v = static_cast<const float*>(p.v);
    a.dout = static_cast<const float*>(p.dout);
    a.dq = static_cast<float*>(p.dq);
    a.dk = static_cast<float*>(p.dk);
    a.dv = static_cast<float*>(p.dv);
    a.offsets = p.offsets;
    a.ntgt = p.num_targets;
    a.num_seqs = p.num_seqs;
    a.heads = p.heads;
    a.row_stride = p.dense ? p.d : (int64_t)p.heads * p.d;
    a.head_stride = p.dense ? p.dense_len * p.d : p.d;
    a.alpha = p.alpha;
    a.dv_scale = 1.0f / p.n;
    a.g_scale = p.alpha / p.n;
    a.ts = p.timestamps;
    a.wpos = p.pos_bias;
    a.wtime = p.time_bias;
    a.gpart = p.rab_partials;
    a.npos = p.num_pos;
    a.ntime = p.num_time;
    a.gstride = RAB ? rab_partial_stride(p.num_pos) : 0;
    a.nparts = RAB_PARTS;
    a.bias_scale = RAB ? (float)(1.0 / (double)p.alpha) : 0.0f;
    using Fn = void (*)(BwdArgsF32);
    const Fn f_dkv = wl.fused ? attn_bwd_dkv_f32<D, true, TGT, RAB>
                              : attn_bwd_dkv_f32<D, false, TGT, RAB>;
    const Fn f_dq = wl.fused ? attn_bwd_dq_f32<D, true, TGT, RAB>
                             : attn_bwd_dq_f32<D, false, TGT, RAB>;
    static int grids[2][2] = {};
    int& g_dkv = grids[wl.fused ? 1 : 0][0];
    int& g_dq = grids[wl.fused ? 1 : 0][1];
    if (!g_dkv) g_dkv = resident_grid(f_dkv, 256);
    if (!g_dq) g_dq = resident_grid(f_dq, 256);
    a.wl = wl;
    hipError_t e;
    if constexpr (RAB) {
        const int64_t cells = (int64_t)RAB_PARTS * a.gstride;
        hipLaunchKernelGGL(rab_zero_kernel, dim3(256), dim3(256), 0, stream, a.gpart, cells);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (start)
        hipExtLaunchKernelGGL(f_dkv, dim3(g_dkv), dim3(256), 0, stream, start, nullptr, 0, a);
    else
        hipLaunchKernelGGL(f_dkv, dim3(g_dkv), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.wl.set = (wl.set + 1) % NSETS;
    hipEvent_t dq_stop = RAB ? nullptr : stop;
    if (dq_stop)
        hipExtLaunchKernelGGL(f_dq, dim3(g_dq), dim3(256), 0, stream, nullptr, dq_stop, 0, a);
    else
        hipLaunchKernelGGL(f_dq, dim3(g_dq), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess || !RAB) return e;
    const int n_out = p.num_pos + p.num_time;
    if (stop)
        hipExtLaunchKernelGGL(rab_reduce_kernel, dim3((n_out + 255) / 256), dim3(256), 0, stream,
                              nullptr, stop, 0, (const float*)a.gpart, a.nparts, a.gstride,
                              p.num_pos, p.num_time, p.d_pos_bias, p.d_time_bias);
    else
        hipLaunchKernelGGL(rab_reduce_kernel, dim3((n_out + 255) / 256), dim3(256), 0, stream,
                           (const float*)a.gpart, a.nparts, a.gstride, p.num_pos, p.num_time,
                           p.d_pos_bias, p.d_time_bias);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_f32(const BwdParams& p, WorkList wl, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
    if (p.timestamps)
        return p.num_targets ? launch_bwd_f32_typed<D, true, true>(p, wl, stream, start, stop)
                             : launch_bwd_f32_typed<D, false, true>(p, wl, stream, start, stop);
    return p.num_targets ? launch_bwd_f32_typed<D, true>(p, wl, stream, start, stop)
                         : launch_bwd_f32_typed<D, false>(p, wl, stream, start, stop);
}

}  // namespace

hipError_t launch_backward(const BwdParams& p, Dtype dt, WorkList wl, hipStream_t stream,
                           hipEvent_t start, hipEvent_t stop) {
    if (dt == Dtype::BF16)
        return p.d == 64 ? launch_bwd_mask<__bf16, 64>(p, wl, stream, start, stop)
                         : launch_bwd_mask<__bf16, 128>(p, wl, stream, start, stop);
    if (dt == Dtype::FP16)
        return p.d == 64 ? launch_bwd_mask<_Float16, 64>(p, wl, stream, start, stop)
                         : launch_bwd_mask<_Float16, 128>(p, wl, stream, start, stop);
    if (dt == Dtype::FP32)
        return p.d == 64 ? launch_bwd_f32<64>(p, wl, stream, start, stop)
                         : launch_bwd_f32<128>(p, wl, stream, start, stop);
    return hipErrorInvalidValue;
}

}  // namespace hstu
