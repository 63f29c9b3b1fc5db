// HSTU jagged causal attention forward on gfx950 matrix cores.
//
//   out[r] = (1/n) * sum_{c <= r} silu(alpha <q_r, k_c>) v_c      (per sequence, head)
//
// (also the target-aware and cached-history masks of M-FALCON, and the dense
// (B, heads, S, d) layout: see MASK_* and the strides in KernelArgs)
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
// built by schedule.hip.  Per item, each wave owns 32 or 64 query rows and
// walks the key/value tiles 0..(last tile that reaches its rows), staged
// through LDS: while tile c is consumed, tiles c+1 and c+2 are in flight from
// HBM.
//
// Transposed products.  With v_mfma_f32_32x32x16_{bf16,f16} a lane's C/D
// registers hold one column and 16 rows of a 32x32 block:
//   column = lane % 32,  row = 8*(r/4) + 4*(lane/32) + r%4   (r = register 0..15).
// Computing S^T = K Q^T (keys down, queries across) therefore leaves each lane
// with one query and 16 keys, which is the k-slice the second product
// O^T = V^T P^T needs in its B operand.  The keys a lane holds for k-step t are
// {16t + 8*(e/4) + 4*(lane/32) + e%4 : e = 0..7}.  For bf16/fp16, V stays
// row-major in LDS and gfx950's transposing LDS read hands each lane exactly
// those keys for its head-dim row of V^T; the fp32 kernel needs no transpose.
//
// Scaling.  With m = -alpha*log2(e)*s, silu(alpha*s) = -(m / log2(e)) *
// 1/(1 + 2^m).  The 16-bit kernel multiplies each Q row by -alpha*log2(e) and
// rounds it to the element type once per item, so the first product yields m
// directly; per score it then forms p = m * rcp(1 + exp2(m)) (two
// transcendental instructions, one add, one multiply) and applies -ln(2)/n to
// the accumulated output once, in the epilogue.  (Rounding the scaled Q adds
// about 2^-9 relative error per bf16 element: measured rel-L2 against the fp64
// definition rises from 2.4e-3 to 2.9e-3 on 4096-token bf16 sequences, and the
// kernel runs 5-6 % faster at d = 64.)  The fp32 kernel scales each score.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"
#include "schedule.h"

namespace hstu {

namespace {

struct KernelArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    const int32_t* offsets;
    const int32_t* ntgt;   // candidates per sequence (target-aware mask), or null
    const uint16_t* kc;    // cached history K, V (MASK_CACHED), or null
    const uint16_t* vc;
    const int32_t* hoff;   // history offsets (MASK_CACHED), or null
    WorkList wl;
    int64_t row_stride;    // elements between consecutive tokens of one head
    int64_t head_stride;   // elements between heads of one token
    int num_seqs;
    int heads;
    float score_scale;  // -alpha * log2(e)
    float out_scale;    // -ln(2) / n
    unsigned long long* clk;   // clock record per workgroup (timed calls), or null
    unsigned clk_id;
};

// The relative-attention-bias kernel's arguments (a separate type, so that
// the other modes' kernels keep their argument block).
struct KernelArgsRab : KernelArgs {
    const int32_t* ts;     // token timestamps (the candidates' with a cached history)
    const int32_t* hts;    // the cached history's timestamps (MASK_RAB_CACHED), or null
    const float* wpos;     // relative attention bias tables
    const float* wtime;
    int npos;              // entries of wpos (distances 0 .. npos-1)
    int ntime;             // entries of wtime (1 .. 32)
    float bias_scale;      // -log2(e): the bias in the scaled scores' units
};

// Which keys a query row sees.
//  CAUSAL : key <= row.
//  TARGETS: the last t tokens of a sequence are candidates that see the
//           history and themselves only: key <= row and (key < hist or
//           key == row), hist = s - t.
//  CACHED : the query rows are candidates whose history K/V come from a
//           cache.  The kernel works on a virtual sequence: the history
//           padded with zero rows to a whole number of key tiles (`hist`
//           keys, read from the cache), then the candidates (read from k, v,
//           rows hist.. of the virtual sequence); the mask is TARGETS' with
//           that hist.  Zero keys and values add exactly nothing.
//  RAB    : CAUSAL, with the relative attention bias added to every score
//           before SiLU (below).
//  RAB_TGT: TARGETS with the bias; M-FALCON (HSTU paper translation, §3.4)
//           adjusts the bias with the mask: a candidate row takes position
//           hist, so its distance to history key c is hist - c and to itself
//           0, while its time gaps use its own timestamp.
//  RAB_CACHED: CACHED with the bias of RAB_TGT: a candidate takes position
//           hlen, the real (unpadded) history length, so its distance to
//           cached key c is hlen - c and to itself 0; the keys' timestamps
//           come from the history's timestamps below the virtual history
//           and from the candidates' above it.
enum : int {
    MASK_CAUSAL = 0,
    MASK_TARGETS = 1,
    MASK_CACHED = 2,
    MASK_RAB = 3,
    MASK_RAB_TGT = 4,
    MASK_RAB_CACHED = 5
};

// Relative attention bias (HSTU paper translation, §3 and Appendix G: a bias
// merging relative position and time, built inside the operator from its
// parameters).  For query row r and key c <= r of a sequence with token
// timestamps ts:
//   rab(r, c) = wpos[r - c] + wtime[min(floor(log2(ts_r - ts_c + 1)), ntime - 1)]
// (wpos[j] = 0 for j >= npos; a negative gap takes the last time bucket).
// floor(log2(x)) = 31 - v_ffbh_u32(x) for x != 0, and v_ffbh_u32(0) = -1 (the
// gap -1), so the kernel keeps a 33-entry LDS table indexed by
// v_ffbh_u32(ts_r + 1 - ts_c) + 1 that already holds the capped bucket's
// entry.  Position entries reach a wave through LDS as well: per key tile, the
// window of wpos that the tile's (row, key) pairs index, staged with the tile.

// Clock record of a timed call: the shader-clock counter and the constant
// 100 MHz counter at a workgroup's start and end (their ratio is the clock the
// workgroup ran at), written by thread 0 with the call's id.
struct ClockMark {
    unsigned long long t, r;
};
__device__ __forceinline__ ClockMark clock_mark(const unsigned long long* clk) {
    ClockMark m = {0, 0};
    if (clk) {
        m.t = __builtin_amdgcn_s_memtime();
        m.r = __builtin_amdgcn_s_memrealtime();
    }
    return m;
}
__device__ __forceinline__ void clock_record(unsigned long long* clk, unsigned id, ClockMark m0) {
    if (clk && threadIdx.x == 0 && blockIdx.x < (unsigned)CLK_SLOTS) {
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        unsigned long long* w = clk + (size_t)CLK_WORDS * blockIdx.x;
        w[0] = m0.t;
        w[1] = m0.r;
        w[2] = t1;
        w[3] = r1;
        w[4] = id;
    }
}

// -log2(e) * silu(alpha*s), given m = -alpha*log2(e)*s.
__device__ __forceinline__ float silu_scaled(float m) {
    const float t = __builtin_amdgcn_exp2f(m);
    return m * __builtin_amdgcn_rcpf(1.0f + t);
}

// ---------------------------------------------------------------------------
// bf16 / fp16 kernel.
//
// Shape: NW waves per workgroup, QB blocks of 32 query rows per wave, key/value
// tiles of BK rows (NKB = BK/32 blocks of 32 keys).  Tiles live in LDS
// unpadded, 16-byte chunks XOR-swizzled by row so that both read patterns are
// free of bank conflicts (measured on gfx950):
//   K (16-byte reads of 32 consecutive rows):      chunk ^ kswz(row)
//   V (transposing 8-byte reads of 4-row groups):   chunk ^ vswz(row)
// Tiles are copied straight from HBM into LDS (16-byte loads whose lanes land
// at consecutive LDS addresses) into NSLOT = PF+1 slots (a K and a V buffer
// each; tile c uses slot c % NSLOT), so tiles c+1 .. c+PF stream in while
// tile c is consumed; one barrier per tile.  Every operand read is a
// lane-constant VGPR plus an immediate offset: the swizzles depend only on
// row bits that 32-key blocks and 16-key steps leave unchanged, and the main
// loop is unrolled over whole slot rotations so that slot, block and step
// offsets are compile-time constants.
//
// A wave's item runs in three phases over the workgroup's tiles:
//   A  tiles whose keys all precede the wave's rows: a software pipeline over
//      32-key blocks, per block b the MFMAs of S(b+1) and of P(b) V are
//      interleaved with the SiLU of S(b);
//   B  tiles holding the wave's diagonal: plain order, scores above the
//      diagonal zeroed before SiLU (silu(0) = 0);
//   C  tiles past the wave's rows: staging and barriers only.
// ---------------------------------------------------------------------------
template <typename T, int D, int NW, int QB, int BK, int PF>
struct Tile16 {
    static constexpr int ROWS_W = 32 * QB;            // query rows per wave
    static constexpr int BQ = NW * ROWS_W;            // query rows per item
    static constexpr int NKB = BK / 32;               // 32-key blocks per tile
    static constexpr int ROW_BYTES = D * 2;           // one K or V row in LDS
    static constexpr int CHUNKS = ROW_BYTES / 16;     // 16-byte chunks per row
    static constexpr int TILE_BYTES = BK * ROW_BYTES;
    static constexpr int NSLOT = PF + 1;                 // tiles in flight: PF
    static constexpr int LDS_BYTES = 2 * NSLOT * TILE_BYTES;
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;   // rows one wave load covers
    static constexpr int LOADS = TILE_BYTES / 1024 / NW;     // loads per wave per tensor
    // Relative attention bias, per wave and slot: 64 key timestamps (BK used),
    // then RAB_WIN entries of wpos, distances wr0 - k0 - BK .. + RAB_WIN - 1.
    static constexpr int RAB_WIN = (ROWS_W + BK + 63) / 64 * 64;
    static constexpr int RAB_WORDS = 64 + RAB_WIN;
    static_assert(LOADS * NW * 1024 == TILE_BYTES, "tile must split into whole wave loads");
    static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(PF >= 2 && (PF - 1) * 2 * LOADS <= 63, "prefetch depth");
    static_assert(LDS_BYTES <= 65536, "LDS reads use 16-bit immediate offsets");
};

// MASK: one of the MASK_* modes; separate instantiations, so that the plain
// causal form carries none of the other modes' registers.
template <int MASK> struct ArgsOf { using type = KernelArgs; };
template <> struct ArgsOf<MASK_RAB> { using type = KernelArgsRab; };
template <> struct ArgsOf<MASK_RAB_TGT> { using type = KernelArgsRab; };
template <> struct ArgsOf<MASK_RAB_CACHED> { using type = KernelArgsRab; };

template <typename T, int D, int NW, int QB, int BK, int PF, bool FUSED, int MASK>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_mfma16(typename ArgsOf<MASK>::type a) {
    constexpr bool CACHED = MASK == MASK_CACHED || MASK == MASK_RAB_CACHED;
    constexpr bool TGT = MASK == MASK_TARGETS || MASK == MASK_RAB_TGT || CACHED;
    // (TGT: hist-based mask)
    constexpr bool RAB = MASK == MASK_RAB || MASK == MASK_RAB_TGT || MASK == MASK_RAB_CACHED;
    // Last-bucket blocks (below) at d = 64 only: at d = 128 the extra path
    // costs the bias kernel some 30-80 more spilled registers.
    constexpr bool FAR = RAB && D == 64;
    using Cfg = Tile16<T, D, NW, QB, BK, PF>;
    using M = Mfma<T>;
    using v8 = typename M::v8;
    using v4 = typename M::v4;
    constexpr int ROWS_W = Cfg::ROWS_W;
    constexpr int BQ = Cfg::BQ;
    constexpr int NKB = Cfg::NKB;
    constexpr int CH = Cfg::CHUNKS;
    constexpr int RB = Cfg::ROW_BYTES;
    constexpr int TB = Cfg::TILE_BYTES;
    constexpr int NKS = D / 16;    // k-steps of the first product
    constexpr int NDB = D / 32;    // 32-wide head-dim blocks of the output

    constexpr int RAB_BYTES = RAB ? Cfg::NSLOT * NW * Cfg::RAB_WORDS * 4 : 0;
    static_assert(!RAB || (PF == 2 && Cfg::RAB_WIN % 64 == 0 && BK <= 64),
                  "bias staging: one tile ahead, whole-wave window loads");
    static_assert(!(RAB && TGT) || QB == 1, "candidate rows: one lane base per item");
    static_assert(Cfg::LDS_BYTES + RAB_BYTES <= 65536, "LDS reads use 16-bit immediate offsets");
    __shared__ __attribute__((aligned(1024))) unsigned char lds[Cfg::LDS_BYTES + RAB_BYTES];
    __shared__ int s_item[NQ];
    __shared__ LocalTables lt;
    __shared__ float ttab[RAB ? 33 : 1];   // time term by v_ffbh_u32(gap + 1) + 1, times -log2(e)
    static_assert(NW * 64 >= FUSE_SEQS && NW * 64 >= 32 * NQ, "fused tables need a thread per sequence");

    const ClockMark clk0 = clock_mark(a.clk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = a.row_stride;        // elements between consecutive tokens
    const int row_bytes = (int)(row_stride * 2);    // bytes between consecutive tokens

    // Lane-constant parts of the addresses.
    // K operand, key block kb, k-step ks: row 32kb + l32, logical chunk 2ks + g.
    const int k_row = l32;
    // V^T operand, 16-key step u, head-dim block db: two transposing reads at
    // rows 16u + 4g + (lane%16)/4 (+8), byte column 2*(32db + 16h + 4(lane%4)).
    const int v_row = 4 * g + ((lane & 15) >> 2);
    const int v_colb = 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    // Tile loads: this wave's load i covers rows (wv + NW*i) * ROWS_PER_LOAD + ...
    int ld_goff[Cfg::LOADS][2];   // [i][K, V] global byte offset inside the tile
#pragma unroll
    for (int i = 0; i < Cfg::LOADS; ++i) {
        const int r = (wv + NW * i) * Cfg::ROWS_PER_LOAD + lane / CH;
        const int pc = lane % CH;
        ld_goff[i][0] = r * row_bytes + 16 * (pc ^ kswz<CH>(r));
        ld_goff[i][1] = r * row_bytes + 16 * (pc ^ vswz<CH>(r));
    }

    // Operand offsets inside a slot.  K row 32kb + l32 has the swizzle of row
    // l32, and V rows 32kb + 16t + v_row (+8) those of rows v_row (+8), so
    // the block and step only add multiples of 32 and 16 rows.
    int k_off[NKS], v_lo[NDB], v_hi[NDB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) k_off[ks] = k_row * RB + 16 * ((2 * ks + g) ^ kswz<CH>(k_row));
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int cb = 64 * db + v_colb;          // byte column inside the row
        v_lo[db] = v_row * RB + 16 * ((cb >> 4) ^ vswz<CH>(v_row)) + (cb & 15);
        v_hi[db] = (v_row + 8) * RB + 16 * ((cb >> 4) ^ vswz<CH>(v_row + 8)) + (cb & 15);
    }
    constexpr int NS = Cfg::NSLOT;
    // Bias staging: this wave's area in slot 0 (byte offsets from the end of
    // the K/V slots) for the key timestamps at 4g, and the lane's window base:
    // the pair (row wr0 + 32qb + l32, key k0 + o) reads window entry
    // 32qb + l32 - o + BK = (l32 - 4g + 5) + 32qb + (RAB_CMAX - o + 4g), where
    // o - 4g = 32kb + 8(r/4) + r%4 <= RAB_CMAX (register r) keeps the rest an
    // immediate offset.
    constexpr int RAB_CMAX = BK - 5;
    const int rab_tk = (wv * Cfg::RAB_WORDS + 4 * g) * 4;
    const int rab_wb = (wv * Cfg::RAB_WORDS + 64 + l32 - 4 * g + 5) * 4;
    // (gap at and above which a pair is in the last time bucket)
    int64_t far_gap = 0;
    if constexpr (RAB) {
        far_gap = ((int64_t)1 << (a.ntime - 1)) - 1;
        if (tid < 33) {
            const int b = tid == 0 ? a.ntime - 1 : min(32 - tid, a.ntime - 1);
            ttab[tid] = a.wtime[b] * a.bias_scale;
        }
    }

    // The tile slots are free until the first item: a fused launch builds its
    // queue tables there and in lt.
    // (Two instantiations, so the compiler knows which memory the tables are
    // in and reads them with LDS or global instructions, not flat ones.)
    Tables tb;
    if constexpr (FUSED)
        tb = build_local_tables(lt, reinterpret_cast<int*>(lds), a.offsets, a.num_seqs, H, BQ,
                                a.wl.ctl);
    else
        tb = global_tables(a.wl);
    clear_sets(a.wl.ctl, a.wl.set + 1, 2);
    ItemSource src(a.wl.ctl, a.wl.set);
    int qx, w;
    while (src.next(tb, s_item, &qx, &w)) {
        const Item it = decode_item(tb, a.num_seqs, H, qx, w);
        const int seq = __builtin_amdgcn_readfirstlane(it.seq);
        const int head = __builtin_amdgcn_readfirstlane(it.head);
        const int qtile = __builtin_amdgcn_readfirstlane(it.qtile);
        const int start = __builtin_amdgcn_readfirstlane(a.offsets[seq]);
        const int len = __builtin_amdgcn_readfirstlane(a.offsets[seq + 1]) - start;
        // s: length of the (virtual) sequence; hist: keys below it are seen
        // by every later row (s for the causal mask); shift: virtual row of
        // the first query row.
        int s = len, hist = len, shift = 0, hstart = 0, hlen = 0;
        if constexpr (MASK == MASK_TARGETS || MASK == MASK_RAB_TGT)
            hist = len - min(max(__builtin_amdgcn_readfirstlane(a.ntgt[seq]), 0), len);
        if constexpr (CACHED) {
            hstart = __builtin_amdgcn_readfirstlane(a.hoff[seq]);
            // (no cache: every history is empty, whatever the offsets say)
            hlen = a.kc ? max(__builtin_amdgcn_readfirstlane(a.hoff[seq + 1]) - hstart, 0) : 0;
            hist = (hlen + BK - 1) / BK * BK;
            shift = hist;
            s = hist + len;
        }
        const int q0 = shift + qtile * BQ;
        const int kv_end = min(s, q0 + BQ);
        const int n_tiles = (kv_end + BK - 1) / BK;
        // Key tiles that hold only candidates below the workgroup's first row
        // are seen by none of its rows: the tile sequence jumps over them.
        // Loop tile c is key tile c below nh and c + jump from there on.
        const int nh = TGT ? (hist + BK - 1) / BK : n_tiles;
        const int jump = TGT ? max(q0 / BK - nh, 0) : 0;
        const int n_iter = n_tiles - jump;
        const int wr0 = q0 + wv * ROWS_W;                // this wave's first query row
        const bool live = wr0 < s;
        // Blocks of 32 keys that are entirely below the wave's first row and
        // the first candidate (unmasked for every row of the wave), and the
        // last block the wave needs.
        const int full_blocks = live ? (TGT ? min(wr0, hist) : wr0) / 32 : 0;
        const int last_block = live ? (min(wr0 + ROWS_W, s) - 1) / 32 : -1;
        const int tiles_a = full_blocks / NKB;             // phase A tiles (all below nh)
        const int last_tile = last_block / NKB;
        const int tiles_ab = live ? (last_tile >= nh ? last_tile - jump : last_tile) + 1 : 0;
        // Sequence i's rows of head h start at off[i] * heads * D + h * head_stride:
        // the jagged (T, heads, D) layout has head_stride D and row stride
        // heads * D, the dense (B, heads, S, D) one (off[i] = i S) S * D and D.
        const int64_t seq_base = (int64_t)start * H * D + (int64_t)head * a.head_stride;

        // Loop tile c into slot c % NS.  The buffer range covers the tile's
        // rows that some row of the workgroup sees (none past kv_end, none
        // past the cached history).
        auto issue_loads = [&](int c) {
            const int kt = c >= nh ? c + jump : c;
            const int k0 = kt * BK;
            // (clamped below by make_rsrc32; min then max, not a clamp, which
            // would become a vector-only instruction and a non-scalar resource)
            const uint16_t* kp;
            const uint16_t* vp;
            int bytes;
            if (CACHED && kt < nh) {
                const int64_t off = ((int64_t)hstart + k0) * row_stride + (int64_t)head * D;
                kp = a.kc + off;
                vp = a.vc + off;
                bytes = min(hlen - k0, BK) * row_bytes;
            } else {
                const int64_t off = seq_base + (int64_t)(k0 - shift) * row_stride;
                kp = a.k + off;
                vp = a.v + off;
                bytes = min(kv_end - k0, BK) * row_bytes;
            }
            const __amdgpu_buffer_rsrc_t rk = make_rsrc32(kp, bytes);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc32(vp, bytes);
            // Computed at run time from an opaque copy of c: with the slot
            // known at compile time the compiler keeps one destination per slot
            // and load in scalar registers, which the kernel does not have.
            int cs = c;
            asm volatile("" : "+s"(cs));
            const int slot = cs % NS;
            // (every read of a slot is ordered by the explicit waits of the
            // prologue, tile_sync and the item's end)
#pragma unroll
            for (int i = 0; i < Cfg::LOADS; ++i) {
                const int dst = (wv + NW * i) * 1024;
                load16_to_lds(rk, lds + slot * TB + dst, ld_goff[i][0]);
                load16_to_lds(rv, lds + (NS + slot) * TB + dst, ld_goff[i][1]);
            }
        };

        // Bias staging through registers: the key timestamps and the wpos
        // window of loop tile c, loaded when the tile's K/V are issued and
        // written to this wave's area of the tile's slot one barrier later.
        uint32_t rab_ts = 0, trp1[QB];
        float rab_w[RAB ? Cfg::RAB_WIN / 64 : 1];
        // The bias sees a candidate row (row >= hist) at position hist, so
        // the window follows the effective rows min(row, hist): the wave's
        // first one, and the lane's lead over it (row - wr0 when causal).
        // With a cached history every row is a candidate at position hlen
        // (the virtual history is padded to whole tiles; hlen is its real
        // length).
        const int wr_eff0 = CACHED ? hlen : TGT ? min(wr0, hist) : wr0;
        const int rab_wb_it = CACHED ? rab_wb - 4 * l32
                              : TGT  ? rab_wb + 4 * (min(wr0 + l32, hist) - wr_eff0 - l32)
                                     : rab_wb;
        // Blocks whose every pair lies in the last time bucket (the keys'
        // latest timestamp at least 2^(ntime-1) - 1 before the wave's
        // earliest row: typical far from the diagonal once the table is
        // shorter than the span of the gaps) take the time term as one
        // constant.  far_mask bit 2 slot + kb marks such a block of the tile
        // in `slot`; rmin is the wave's earliest row timestamp.
        uint32_t far_mask = 0;
        int rmin = 0;
        auto issue_rab = [&](int c) {
            if constexpr (RAB) {
                const int k0 = (TGT && c >= nh ? c + jump : c) * BK;
                // (with a cached history: the history's timestamps below the
                // virtual history, padding rows reading 0, then the candidates')
                const __amdgpu_buffer_rsrc_t rts =
                        !CACHED ? make_rsrc32(a.ts + start + k0, min(kv_end - k0, BK) * 4)
                        : k0 < hist
                                ? make_rsrc32(a.hts + hstart + k0, min(hlen - k0, BK) * 4)
                                : make_rsrc32(a.ts + start + (k0 - shift), min(kv_end - k0, BK) * 4);
                rab_ts = __builtin_amdgcn_raw_buffer_load_b32(rts, lane * 4, 0, 0);
                const __amdgpu_buffer_rsrc_t rp = make_rsrc32(a.wpos, a.npos * 4);
                // Negative distances belong to masked pairs only (they read
                // as zero), except under the target-aware mask, where a
                // candidate's own key, at distance hist - row <= 0 from the
                // row's effective position hist, takes distance 0: there they
                // read wpos[0].
                const int jw0 = wr_eff0 - k0 - BK;
#pragma unroll
                for (int u = 0; u < Cfg::RAB_WIN / 64; ++u)
                    rab_w[u] = __builtin_bit_cast(
                            float, __builtin_amdgcn_raw_buffer_load_b32(
                                           rp, 4 * (TGT ? max(jw0 + lane + 64 * u, 0)
                                                        : jw0 + lane + 64 * u),
                                           0, 0));
            }
        };
        auto rab_store = [&](int c) {
            if constexpr (RAB) {
                float* area = reinterpret_cast<float*>(lds + Cfg::LDS_BYTES) +
                              ((c % NS) * NW + wv) * Cfg::RAB_WORDS;
                area[lane] = __builtin_bit_cast(float, rab_ts);
#pragma unroll
                for (int u = 0; u < Cfg::RAB_WIN / 64; ++u)
                    area[64 + 64 * u + lane] = rab_w[u] * a.bias_scale;
                // latest key timestamp of each 32-key block (lanes past the
                // tile or the sequence read 0, which can only make a block
                // look nearer)
                // (the maximum within each 16-lane row by DPP: quad
                // permutations xor 1 and xor 2, then the half-row and row
                // mirrors; a block's is the larger of its two rows')
                if constexpr (FAR) {
                    int m = (int)rab_ts;
                    m = max(m, __builtin_amdgcn_update_dpp(m, m, 0xB1, 0xF, 0xF, false));
                    m = max(m, __builtin_amdgcn_update_dpp(m, m, 0x4E, 0xF, 0xF, false));
                    m = max(m, __builtin_amdgcn_update_dpp(m, m, 0x141, 0xF, 0xF, false));
                    m = max(m, __builtin_amdgcn_update_dpp(m, m, 0x140, 0xF, 0xF, false));
                    const int sh = 2 * (c % NS);
                    uint32_t bits = 0;
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const int kmax = max(__builtin_amdgcn_readlane(m, 32 * kb),
                                             __builtin_amdgcn_readlane(m, 32 * kb + 16));
                        if ((int64_t)rmin - kmax >= far_gap) bits |= 1u << kb;
                    }
                    far_mask = (far_mask & ~(3u << sh)) | (bits << sh);
                }
            }
        };
        if constexpr (RAB) {
            const __amdgpu_buffer_rsrc_t rt =
                    make_rsrc(a.ts + start + (wr0 - shift), (int64_t)(s - wr0) * 4);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                trp1[qb] = __builtin_amdgcn_raw_buffer_load_b32(rt, (qb * 32 + l32) * 4, 0, 0) + 1u;
        }

        // Q^T operand: query rows wr0 + 32*qb + l32, head-dim slice [16ks + 8g, +8).
        v8 qop[QB][NKS];
        {
            const __amdgpu_buffer_rsrc_t rq =
                    make_rsrc(a.q + seq_base + (int64_t)(wr0 - shift) * row_stride,
                              (int64_t)(s - wr0) * row_bytes);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    qop[qb][ks] = __builtin_bit_cast(
                            v8, __builtin_amdgcn_raw_buffer_load_b128(
                                        rq, (qb * 32 + l32) * row_bytes + (ks * 16 + g * 8) * 2, 0, 0));
            // Q * (-alpha * log2(e)), rounded to the element type (nearest even)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    qop[qb][ks] = __builtin_convertvector(
                            __builtin_convertvector(qop[qb][ks], f32x8) * a.score_scale, v8);
        }
        f32x16 o[NDB][QB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[db][qb] = (f32x16){};

        // ---- building blocks ------------------------------------------------
        // Initial value of the S^T accumulators for key block kb of the tile
        // in `slot`: zero, or with the bias, -log2(e) rab (so that with the
        // scaled Q the accumulator ends at -log2(e) (alpha <q, k> + rab)).  Register
        // r of lane (l32, g) is key 32kb + 8(r/4) + 4g + r%4 of query row
        // wr0 + 32qb + l32.
        auto acc_init = [&](int slot, int kb, f32x16* acc) {
            if constexpr (RAB) {
                const unsigned char* ra = lds + Cfg::LDS_BYTES + slot * NW * Cfg::RAB_WORDS * 4;
                if (FAR && ((far_mask >> (2 * slot + kb)) & 1u)) {
                    const float tlast = ttab[0];   // the last bucket's entry
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
                            acc[qb][r] = *reinterpret_cast<const float*>(
                                                 ra + rab_wb_it + 4 * (32 * qb + RAB_CMAX - o)) +
                                         tlast;
                        }
                    return;
                }
                u32x4 tk[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    tk[j] = *reinterpret_cast<const u32x4*>(ra + rab_tk + 4 * (32 * kb + 8 * j));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
                        const float bp = *reinterpret_cast<const float*>(
                                ra + rab_wb_it + 4 * (32 * qb + RAB_CMAX - o));
                        const uint32_t x = trp1[qb] - tk[r >> 2][r & 3];
                        int f;
                        asm("v_ffbh_u32 %0, %1" : "=v"(f) : "v"(x));
                        acc[qb][r] = bp + ttab[f + 1];
                    }
            }
        };
        // S^T for key block kb of the tile in `slot` into st[qb].
        auto qk = [&](int slot, int kb, f32x16* st) {
            const unsigned char* kl = lds + slot * TB + kb * 32 * RB;
            if constexpr (RAB) {
                acc_init(slot, kb, st);
            } else {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) st[qb] = (f32x16){};
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const v8 ka = *reinterpret_cast<const v8*>(kl + k_off[ks]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) st[qb] = M::mma(ka, qop[qb][ks], st[qb]);
            }
        };
        // Weights for the 16-key step t of a block (registers 8t .. 8t+7).
        auto weights = [&](const f32x16* st, int t, v8* pb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                f32x8 pf;
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[e] = silu_scaled(st[qb][8 * t + e]);
                pb[qb] = __builtin_convertvector(pf, v8);
            }
        };
        // O^T += V^T P^T for the 16-key step t of key block kb in `slot`.
        auto pv = [&](int slot, int kb, int t, const v8* pb) {
            const unsigned char* vl = lds + (NS + slot) * TB + (kb * 32 + 16 * t) * RB;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const i16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vl + v_lo[db]));
                const i16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vl + v_hi[db]));
                const v8 va = __builtin_bit_cast(
                        v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[db][qb] = M::mma(va, pb[qb], o[db][qb]);
            }
        };
        // Operand reads and the second product, for the pipelined body.
        auto kread = [&](int slot, int kb, int ks) -> v8 {
            return *reinterpret_cast<const v8*>(lds + slot * TB + kb * 32 * RB + k_off[ks]);
        };
        auto vread = [&](int slot, int kb, int t, int db) -> v8 {
            const unsigned char* vl = lds + (NS + slot) * TB + (kb * 32 + 16 * t) * RB;
            const i16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vl + v_lo[db]));
            const i16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vl + v_hi[db]));
            return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        auto mma_pv = [&](const v8* va, const v8* pb) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[db][qb] = M::mma(va[db], pb[qb], o[db][qb]);
        };
        // Block b on or past the diagonal, or holding candidate keys: scores
        // of keys a row does not see are zeroed (silu(0) = 0).  Register r of
        // lane (l32, g) holds key 32b + 8(r/4) + 4g + r%4 of query row
        // wr0 + 32qb + l32, which sees it iff key <= row and (key < hist or
        // key == row).
        auto masked_block = [&](int slot, int kb, int b) {
            f32x16 st[QB];
            qk(slot, kb, st);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // offsets from the lane's first key: the row itself, and the
                // bound below which keys are seen (min(row, hist); the
                // condition above is key == row or key < min(row, hist))
                const int eq = wr0 + 32 * qb + l32 - 32 * b - 4 * g;
                if constexpr (TGT) {
                    const int lt = min(wr0 + 32 * qb + l32, hist) - 32 * b - 4 * g;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int o = 8 * (r >> 2) + (r & 3);
                        st[qb][r] = (o < lt || o == eq) ? st[qb][r] : 0.0f;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        st[qb][r] = (8 * (r >> 2) + (r & 3) <= eq) ? st[qb][r] : 0.0f;
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                v8 pb[QB];
                weights(st, t, pb);
                pv(slot, kb, t, pb);
            }
        };

        // ---- prologue: tiles 0 .. PF-1 in flight, wait for tile 0 -------------
        // Tiles are always issued PF ahead, also past the sequence (their buffer
        // range is empty, so they read nothing), which keeps the number of loads
        // in flight after tile c+1 fixed: a wait on the load counter then
        // covers exactly the tiles up to c+1.  Loads return in issue order.
        if constexpr (RAB) {
            // (tile 0's bias values are written once its loads are in; tile
            // 1's are loaded then, and written at the first barrier)
            issue_loads(0);
            issue_rab(0);
#pragma unroll
            for (int c = 1; c < PF; ++c) issue_loads(c);
            __builtin_amdgcn_s_waitcnt(VMCNT_LE((PF - 1) * 2 * Cfg::LOADS));
            if constexpr (FAR) {
                int t = 0x7fffffff;   // rows past the sequence do not count
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    if (wr0 + 32 * qb + l32 < s) t = min(t, (int)(trp1[qb] - 1u));
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) t = min(t, __shfl_xor(t, off));
                rmin = __builtin_amdgcn_readfirstlane(t);
            }
            rab_store(0);
            issue_rab(1);
        } else {
#pragma unroll
            for (int c = 0; c < PF; ++c) issue_loads(c);
            __builtin_amdgcn_s_waitcnt(VMCNT_LE((PF - 1) * 2 * Cfg::LOADS));
        }
        __syncthreads();

        // One barrier per tile.  At barrier c every wave has finished its loads
        // of tile c+1 and every read of tile c-1 (slot (c+PF) % NS); then tile
        // c+PF is issued into that slot.
        //
        // Two workgroups share each CU, and the SIMDs favour the older of two
        // ready waves, so left alone one workgroup runs at nearly its solo
        // speed and the other takes the leftover issue slots.  The wave
        // priority alternates every two tiles, in opposite phase for the two
        // halves of the grid (the dispatcher fills every CU once with the
        // first half before placing the second), so the two share the SIMDs
        // more evenly and finish their items closer together (measured 1.5 %
        // faster on 16 x 4096, 3 % on 8 x 8k-20k).
        auto tile_sync = [&](int c) {
            __builtin_amdgcn_s_waitcnt(VMCNT_LE((PF - 2) * 2 * Cfg::LOADS));
            if constexpr (RAB) rab_store(c + 1);
            __syncthreads();
            issue_loads(c + PF);
            if constexpr (RAB) issue_rab(c + PF);
            if ((((c >> 1) + (blockIdx.x >= gridDim.x / 2 ? 1 : 0)) & 1) != 0)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        };

        // ---- phase A: pipelined full blocks -----------------------------------
        // Body of block b: the SiLU of S(b) on the vector ALUs while the matrix
        // cores run S(b+1) and P(b) V.  All operands of the body are read from
        // LDS first; the SiLU of the first 16 keys overlaps the products of the
        // previous block's last 16 keys and S(b+1), the SiLU of the last 16
        // keys overlaps P V of the first 16; the product of the last 16 keys
        // waits for the next body (so no product has to wait for the SiLU right
        // before it), and S(b+1) is complete well before the next body's SiLU
        // reads it.  Tile c's
        // barrier comes right before the body of its last block, the first body
        // that reads tile c+1 (its K).  Two score arrays alternate by block
        // parity, so nothing is copied.  The main loop
        // runs GT tiles per trip (whole slot rotations, an even number of
        // blocks), so every slot, block and parity is a constant in the unrolled
        // code; the remaining tiles take the same body with computed slots.  The
        // last body also computes S of the first block past phase A, which
        // phase B computes again with its mask (that tile is loaded: it holds
        // the wave's diagonal).
        constexpr int GT = (NS * NKB) % 2 == 0 ? NS : 2 * NS;
        f32x16 sc[2][QB];
        v8 p1d[QB], v1d[NDB];   // deferred: weights and V^T of the last block's keys 16..31
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) p1d[qb] = (v8){};
#pragma unroll
        for (int db = 0; db < NDB; ++db) v1d[db] = (v8){};
        auto body = [&](int slot, int kb, int next_slot, int next_kb, bool sync, int c,
                        f32x16* cur, f32x16* nxt) {
            // (the compiler's exp/MFMA interleaving strategy for this block:
            // measured 0.5-1 % faster than its default schedule)
            __builtin_amdgcn_iglp_opt(2);
            if (sync) tile_sync(c);
            v8 ka[NKS], va0[NDB], va1[NDB];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) ka[ks] = kread(next_slot, next_kb, ks);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                va0[db] = vread(slot, kb, 0, db);
                va1[db] = vread(slot, kb, 1, db);
            }
            v8 p0[QB], p1[QB];
            weights(cur, 0, p0);
            mma_pv(v1d, p1d);
            if constexpr (RAB) {
                acc_init(next_slot, next_kb, nxt);
            } else {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) nxt[qb] = (f32x16){};
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) nxt[qb] = M::mma(ka[ks], qop[qb][ks], nxt[qb]);
            weights(cur, 1, p1);
            mma_pv(va0, p0);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) p1d[qb] = p1[qb];
#pragma unroll
            for (int db = 0; db < NDB; ++db) v1d[db] = va1[db];
        };
        if (tiles_a > 0) {
            qk(0, 0, sc[0]);
            const int groups = tiles_a / GT;
            for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
                for (int j = 0; j < GT; ++j)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const int par = (j * NKB + kb) & 1;
                        const bool last = kb == NKB - 1;
                        body(j % NS, kb, last ? (j + 1) % NS : j % NS, last ? 0 : kb + 1, last,
                             gi * GT + j, sc[par], sc[par ^ 1]);
                    }
            }
            const int nA = tiles_a * NKB;
            auto body_at = [&](int b, f32x16* cur, f32x16* nxt) {
                const int c = b / NKB, kb = b % NKB, bn = b + 1;
                body(c % NS, kb, (bn / NKB) % NS, bn % NKB, kb == NKB - 1, c, cur, nxt);
            };
            for (int b = groups * GT * NKB; b < nA; b += 2) {
                body_at(b, sc[0], sc[1]);
                if (b + 1 < nA) body_at(b + 1, sc[1], sc[0]);
            }
            mma_pv(v1d, p1d);   // the last block's keys 16..31
        }
        int c = tiles_a;
        // ---- phase B: the tiles holding the wave's diagonal (and the first -----
        // candidate) ------------------------------------------------------------
        // Plain order; the barrier comes after the tile's blocks, since the
        // last one still reads this tile's K.
        for (; c < tiles_ab; ++c) {
            const int slot = c % NS;
            const int kt = c >= nh ? c + jump : c;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int b = kt * NKB + kb;
                if (b < full_blocks) {
                    f32x16 st[QB];
                    qk(slot, kb, st);
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        v8 pb[QB];
                        weights(st, t, pb);
                        pv(slot, kb, t, pb);
                    }
                } else if (b <= last_block && (!TGT || 32 * b < hist || 32 * b + 31 >= wr0)) {
                    // (blocks of candidate keys below the wave's rows are seen
                    // by none of them)
                    masked_block(slot, kb, b);
                }
            }
            tile_sync(c);
        }
        // ---- phase C: staging only --------------------------------------------
        for (; c < n_iter; ++c) tile_sync(c);
        __builtin_amdgcn_s_waitcnt(VMCNT_LE(0));   // nothing left landing in LDS

        // Epilogue: lane holds query wr0 + 32*qb + l32 and head-dim rows
        // 32*db + 8*i + 4*g + (0..3).  Stores past the sequence are dropped.
        if (live) {
            const __amdgpu_buffer_rsrc_t ro =
                    make_rsrc(a.out + seq_base + (int64_t)(wr0 - shift) * row_stride,
                              (int64_t)(s - wr0) * row_bytes);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        f32x4 x;
#pragma unroll
                        for (int j = 0; j < 4; ++j) x[j] = o[db][qb][4 * i + j] * a.out_scale;
                        const v4 y = __builtin_convertvector(x, v4);
                        __builtin_amdgcn_raw_buffer_store_b64(
                                __builtin_bit_cast(u32x2, y), ro,
                                (qb * 32 + l32) * row_bytes + (db * 32 + 8 * i + 4 * g) * 2, 0, 0);
                    }
        }
    }
    clock_record(a.clk, a.clk_id, clk0);
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
    // K rows hold a row's even features, then its odd ones (the two k-slices
    // the lane halves read), so a lane reads four k-steps' operands with one
    // 16-byte read; V is held transposed (a head-dim row per feature, keys
    // along it), so one 16-byte read gives four keys' operands.  Strides in
    // floats, multiples of 4 with 4 mod 32, which spreads 16-byte reads of
    // consecutive rows over the banks.
    static constexpr int KSTR = D + 4;
    static constexpr int VTSTR = BK + 4;
    static constexpr int CHUNKS = BK * D / 4 / THREADS;  // 16-byte loads per thread per tensor
    static_assert(CHUNKS * THREADS * 4 == BK * D, "tile must split evenly");
};

struct KernelArgsF32 {
    const float* q;
    const float* k;
    const float* v;
    float* out;
    const int32_t* offsets;
    const int32_t* ntgt;   // candidates per sequence (target-aware mask), or null
    const float* kc;       // cached history K, V, or null
    const float* vc;
    const int32_t* hoff;   // history offsets: the cached-history form when non-null
    const int32_t* ts;     // token timestamps: the relative attention bias when non-null
    const int32_t* hts;    // the cached history's timestamps (bias with a cached history)
    const float* wpos;
    const float* wtime;
    int npos;
    int ntime;
    WorkList wl;
    int64_t row_stride;
    int64_t head_stride;
    int num_seqs;
    int heads;
    float score_scale;
    float out_scale;
    unsigned long long* clk;   // clock record per workgroup (timed calls), or null
    unsigned clk_id;
};

template <int D, int NW, int BK, bool FUSED>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_mfma_f32(KernelArgsF32 a) {
    using Cfg = TileF32<D, NW, BK>;
    constexpr int BQ = Cfg::BQ;
    __shared__ __attribute__((aligned(16))) float kl[BK * Cfg::KSTR];
    __shared__ __attribute__((aligned(16))) float vt[D * Cfg::VTSTR];
    __shared__ int s_item[NQ];
    __shared__ LocalTables lt;
    static_assert(NW * 64 >= FUSE_SEQS && NW * 64 >= 32 * NQ, "fused tables need a thread per sequence");

    const ClockMark clk0 = clock_mark(a.clk);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int g = lane >> 5;
    const int l32 = lane & 31;
    const int H = a.heads;
    const int64_t row_stride = a.row_stride;

    Tables tb;
    if constexpr (FUSED)
        tb = build_local_tables(lt, reinterpret_cast<int*>(kl), a.offsets, a.num_seqs, H, BQ,
                                a.wl.ctl);
    else
        tb = global_tables(a.wl);
    clear_sets(a.wl.ctl, a.wl.set + 1, 2);
    ItemSource src(a.wl.ctl, a.wl.set);
    int qx, w;
    while (src.next(tb, s_item, &qx, &w)) {
        const Item it = decode_item(tb, a.num_seqs, H, qx, w);
        // Virtual sequence, key-tile jump and mask as in the 16-bit kernel.
        const int start = a.offsets[it.seq];
        const int len = a.offsets[it.seq + 1] - start;
        int s = len, hist = len, shift = 0, hstart = 0, hlen = 0;
        if (a.hoff) {
            hstart = a.hoff[it.seq];
            // (no cache: every history is empty, whatever the offsets say)
            hlen = a.kc ? max(a.hoff[it.seq + 1] - hstart, 0) : 0;
            hist = (hlen + BK - 1) / BK * BK;
            shift = hist;
            s = hist + len;
        } else if (a.ntgt) {
            hist = len - min(max(a.ntgt[it.seq], 0), len);
        }
        const int q0 = shift + it.qtile * BQ;
        const int kv_end = min(s, q0 + BQ);
        const int n_tiles = (kv_end + BK - 1) / BK;
        const int nh = (hist + BK - 1) / BK;
        const int jump = max(q0 / BK - nh, 0);
        const int wr0 = q0 + wv * 32;
        const bool wave_live = wr0 < s;
        const int my_row = wr0 + l32;
        const int64_t seq_base = (int64_t)start * H * D + (int64_t)it.head * a.head_stride;
        // relative attention bias: this row's timestamp + 1, and the position
        // its distances are taken from (a candidate sits right after the
        // history: hlen with a cached history, hist under the target-aware mask)
        const uint32_t trp1 =
                (a.ts && my_row < s) ? (uint32_t)a.ts[start + my_row - shift] + 1u : 0u;
        const int pos_row = a.hoff ? hlen : min(my_row, hist);

        float qf[D / 2];
        {
            const float* qp = a.q + seq_base + (int64_t)(my_row - shift) * row_stride;
#pragma unroll
            for (int ks = 0; ks < D / 2; ++ks) qf[ks] = (my_row < s) ? qp[2 * ks + g] : 0.0f;
        }
        f32x16 o[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = (f32x16){};

        // Tile c's K and V into registers (this thread's chunks), and from
        // there into LDS: the loads of tile c + 1 are in flight while tile c
        // is computed.
        const int n_iter = n_tiles - jump;
        float4 pk[Cfg::CHUNKS], pv[Cfg::CHUNKS];
        auto fetch = [&](int c) {
            const int k0 = (c >= nh ? c + jump : c) * BK;
            const bool from_cache = a.hoff && k0 < hist;
#pragma unroll
            for (int i = 0; i < Cfg::CHUNKS; ++i) {
                const int id = tid + i * Cfg::THREADS;
                const int r = id / (D / 4), c4 = id % (D / 4);
                float4 xk = make_float4(0.f, 0.f, 0.f, 0.f), xv = xk;
                if (from_cache) {
                    if (k0 + r < hlen) {
                        const int64_t off = ((int64_t)hstart + k0 + r) * row_stride +
                                            (int64_t)it.head * D + c4 * 4;
                        xk = *reinterpret_cast<const float4*>(a.kc + off);
                        xv = *reinterpret_cast<const float4*>(a.vc + off);
                    }
                } else if (k0 + r < kv_end) {
                    const int64_t off =
                            seq_base + (int64_t)(k0 - shift + r) * row_stride + c4 * 4;
                    xk = *reinterpret_cast<const float4*>(a.k + off);
                    xv = *reinterpret_cast<const float4*>(a.v + off);
                }
                pk[i] = xk;
                pv[i] = xv;
            }
        };
        if (n_iter > 0) fetch(0);
        for (int c = 0; c < n_iter; ++c) {
            const int k0 = (c >= nh ? c + jump : c) * BK;
#pragma unroll
            for (int i = 0; i < Cfg::CHUNKS; ++i) {
                const int id = tid + i * Cfg::THREADS;
                const int r = id / (D / 4), c4 = id % (D / 4);
                // features 4 c4 .. 4 c4 + 3: the even ones to 2 c4, 2 c4 + 1,
                // the odd ones to D/2 + 2 c4, D/2 + 2 c4 + 1
                float* kd = kl + r * Cfg::KSTR;
                *reinterpret_cast<float2*>(kd + 2 * c4) = make_float2(pk[i].x, pk[i].z);
                *reinterpret_cast<float2*>(kd + D / 2 + 2 * c4) = make_float2(pk[i].y, pk[i].w);
                float* vd = vt + 4 * c4 * Cfg::VTSTR + r;
                vd[0] = pv[i].x;
                vd[Cfg::VTSTR] = pv[i].y;
                vd[2 * Cfg::VTSTR] = pv[i].z;
                vd[3 * Cfg::VTSTR] = pv[i].w;
            }
            __syncthreads();
            if (c + 1 < n_iter) fetch(c + 1);
            // Skip tiles no row of the wave sees: past its last row, or all
            // candidate keys below its first row.
            const bool skip = !wave_live || k0 > wr0 + 31 || (k0 >= hist && k0 + BK - 1 < wr0);
            if (!skip) {
                const bool partial = k0 + BK - 1 > wr0 || k0 + BK > hist;
#pragma unroll
                for (int kb = 0; kb < BK / 32; ++kb) {
                    f32x16 st = (f32x16){};
                    // k-step ks takes feature 2 ks + g of key row kb*32 + l32
                    const float* krow = kl + (kb * 32 + l32) * Cfg::KSTR + g * (D / 2);
#pragma unroll
                    for (int j = 0; j < D / 8; ++j) {
                        const float4 kv = *reinterpret_cast<const float4*>(krow + 4 * j);
                        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, qf[4 * j], st, 0, 0, 0);
                        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, qf[4 * j + 1], st, 0, 0, 0);
                        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, qf[4 * j + 2], st, 0, 0, 0);
                        st = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, qf[4 * j + 3], st, 0, 0, 0);
                    }
                    // Registers 4 rq .. 4 rq + 3 hold keys kb*32 + 8 rq + 4 g + 0..3:
                    // one 16-byte read of V^T per head-dim block feeds their
                    // four k-steps of the second product.
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        // The exp2 argument of each pair; one the row does not
                        // see gets +2^100, whose weight m / (1 + 2^m) comes out
                        // as 0.  (Each run-time choice is taken once per four
                        // keys, not per key, so the SiLU of the four is
                        // straight-line code.)
                        float m[4];
                        if (a.ts) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int key = k0 + kb * 32 + 8 * rq + 4 * g + i;
                                // (a candidate row sits at position hist; its own
                                // key at distance 0)
                                const int dist = key == my_row ? 0 : pos_row - key;
                                float bias = (dist >= 0 && dist < a.npos) ? a.wpos[dist] : 0.0f;
                                // key timestamp: the cached history's below hist
                                // (its padding, masked by zero V, reads none)
                                uint32_t tk = 0u;
                                if (a.hoff && key < hist)
                                    tk = key < hlen ? (uint32_t)a.hts[hstart + key] : 0u;
                                else if (key < s)
                                    tk = (uint32_t)a.ts[start + key - shift];
                                const uint32_t x = trp1 - tk;
                                const int lz = __clz((int)x);   // 32 for x == 0 (gap -1)
                                bias += a.wtime[lz == 32 ? a.ntime - 1
                                                         : min(31 - lz, a.ntime - 1)];
                                m[i] = __builtin_fmaf(st[4 * rq + i], a.score_scale, bias * -LOG2E);
                            }
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) m[i] = st[4 * rq + i] * a.score_scale;
                        }
                        if (partial) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int key = k0 + kb * 32 + 8 * rq + 4 * g + i;
                                m[i] = (key <= my_row && (key < hist || key == my_row)) ? m[i]
                                                                                      : 0x1p100f;
                            }
                        }
                        float p4[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) p4[i] = silu_scaled(m[i]);
#pragma unroll
                        for (int db = 0; db < D / 32; ++db) {
                            const float4 vv = *reinterpret_cast<const float4*>(
                                    vt + (db * 32 + l32) * Cfg::VTSTR + kb * 32 + 8 * rq + 4 * g);
                            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.x, p4[0], o[db], 0, 0, 0);
                            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.y, p4[1], o[db], 0, 0, 0);
                            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.z, p4[2], o[db], 0, 0, 0);
                            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.w, p4[3], o[db], 0, 0, 0);
                        }
                    }
                }
            }
            __syncthreads();
        }

        if (my_row < s) {
            float* op = a.out + seq_base + (int64_t)(my_row - shift) * row_stride;
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
    clock_record(a.clk, a.clk_id, clk0);
}

// ---------------------------------------------------------------------------
// Launch configuration per (element type, head size).
// ---------------------------------------------------------------------------
constexpr int NW16 = 4;
template <int D> struct QBlocks { static constexpr int value = D == 64 ? 2 : 1; };
// The cached-history form runs one 32-row block per wave (128-row items): its
// calls hold one micro-batch of candidates per request, and 256-row items
// would leave half of the resident workgroups without work at 16 x 1024.  So
// does the relative-attention-bias form, whose bias terms need the registers
// a second block would take.
template <int D, int MASK> struct QBlocksFor {
    static constexpr int value =
            MASK == MASK_CACHED || MASK == MASK_RAB || MASK == MASK_RAB_TGT ||
                            MASK == MASK_RAB_CACHED
                    ? 1
                    : QBlocks<D>::value;
};
template <int D> struct KeyTile { static constexpr int value = D == 64 ? 64 : 32; };
// Key tiles in flight: two at d = 64; three at d = 128, whose 32-key tiles
// hold less work per wait (measured 3 % faster on 4096 sequences of 1-256
// tokens, the same on the others; at d = 64 a third tile measured no gain).
// The bias forms stage their tables one tile ahead and keep two.
template <int D> struct Prefetch { static constexpr int value = D == 64 ? 2 : 3; };
constexpr int PF_RAB = 2;
constexpr int NWF = 4;
constexpr int BKF = 32;

template <typename T, int D>
hipError_t launch16(const FwdParams& p, WorkList wl, int grid, hipStream_t stream, hipEvent_t start,
                  hipEvent_t stop) {
    KernelArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.out = static_cast<uint16_t*>(p.out);
    a.offsets = p.offsets;
    a.ntgt = p.num_targets;
    a.kc = static_cast<const uint16_t*>(p.k_cache);
    a.vc = static_cast<const uint16_t*>(p.v_cache);
    a.hoff = p.hist_offsets;
    a.row_stride = p.dense ? p.d : (int64_t)p.heads * p.d;
    a.head_stride = p.dense ? p.dense_len * p.d : p.d;
    a.wl = wl;
    a.num_seqs = p.num_seqs;
    a.heads = p.heads;
    a.score_scale = -p.alpha * LOG2E;
    a.out_scale = -LN2 / p.n;
    a.clk = p.clk;
    a.clk_id = p.clk_id;
    constexpr int QB = QBlocks<D>::value, BK = KeyTile<D>::value, PF = Prefetch<D>::value;
    constexpr int QBC = QBlocksFor<D, MASK_CACHED>::value;
    if (p.timestamps) {
        KernelArgsRab ar;
        static_cast<KernelArgs&>(ar) = a;
        ar.ts = p.timestamps;
        ar.hts = p.hist_timestamps;
        ar.wpos = p.pos_bias;
        ar.wtime = p.time_bias;
        ar.npos = p.num_pos;
        ar.ntime = p.num_time;
        // (the bias joins the scores in the accumulators, in the units of
        // the scaled Q: rab * (-log2(e)))
        ar.bias_scale = -LOG2E;
        constexpr int QBR = QBlocksFor<D, MASK_RAB>::value;
        static_assert(QBlocksFor<D, MASK_RAB_TGT>::value == QBR &&
                              QBlocksFor<D, MASK_RAB_CACHED>::value == QBR &&
                              QBlocksFor<D, MASK_CACHED>::value == QBR,
                      "one item shape for the bias forms and the cached history");
        using FnR = void (*)(KernelArgsRab);
        static constexpr FnR fnr[2][3] = {
                {attn_fwd_mfma16<T, D, NW16, QBR, BK, PF_RAB, false, MASK_RAB>,
                 attn_fwd_mfma16<T, D, NW16, QBR, BK, PF_RAB, false, MASK_RAB_TGT>,
                 attn_fwd_mfma16<T, D, NW16, QBR, BK, PF_RAB, false, MASK_RAB_CACHED>},
                {attn_fwd_mfma16<T, D, NW16, QBR, BK, PF_RAB, true, MASK_RAB>,
                 attn_fwd_mfma16<T, D, NW16, QBR, BK, PF_RAB, true, MASK_RAB_TGT>,
                 attn_fwd_mfma16<T, D, NW16, QBR, BK, PF_RAB, true, MASK_RAB_CACHED>}};
        const int tg = p.hist_offsets ? 2 : p.num_targets ? 1 : 0;
        const FnR fn = fnr[wl.fused ? 1 : 0][tg];
        if (grid <= 0) {
            static int cached[2][3] = {};
            int& c = cached[wl.fused ? 1 : 0][tg];
            if (!c) c = resident_grid(fn, NW16 * 64);
            grid = c;
        }
        if (start)
            hipExtLaunchKernelGGL(fn, dim3(grid), dim3(NW16 * 64), 0, stream, start, stop, 0, ar);
        else
            hipLaunchKernelGGL(fn, dim3(grid), dim3(NW16 * 64), 0, stream, ar);
        return hipGetLastError();
    }
    const int mode = p.hist_offsets ? MASK_CACHED : p.num_targets ? MASK_TARGETS : MASK_CAUSAL;
    using Fn = void (*)(KernelArgs);
    static constexpr Fn fns[2][3] = {
            {attn_fwd_mfma16<T, D, NW16, QB, BK, PF, false, MASK_CAUSAL>,
             attn_fwd_mfma16<T, D, NW16, QB, BK, PF, false, MASK_TARGETS>,
             attn_fwd_mfma16<T, D, NW16, QBC, BK, PF, false, MASK_CACHED>},
            {attn_fwd_mfma16<T, D, NW16, QB, BK, PF, true, MASK_CAUSAL>,
             attn_fwd_mfma16<T, D, NW16, QB, BK, PF, true, MASK_TARGETS>,
             attn_fwd_mfma16<T, D, NW16, QBC, BK, PF, true, MASK_CACHED>}};
    const Fn fn = fns[wl.fused ? 1 : 0][mode];
    if (grid <= 0) {
        static int cached[2][3] = {};
        int& c = cached[wl.fused ? 1 : 0][mode];
        if (!c) c = resident_grid(fn, NW16 * 64);
        grid = c;
    }
    if (start)
        hipExtLaunchKernelGGL(fn, dim3(grid), dim3(NW16 * 64), 0, stream, start, stop, 0, a);
    else
        hipLaunchKernelGGL(fn, dim3(grid), dim3(NW16 * 64), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const FwdParams& p, WorkList wl, int grid, hipStream_t stream, hipEvent_t start,
                  hipEvent_t stop) {
    KernelArgsF32 a;
    a.q = static_cast<const float*>(p.q);
    a.k = static_cast<const float*>(p.k);
    a.v = static_cast<const float*>(p.v);
    a.out = static_cast<float*>(p.out);
    a.offsets = p.offsets;
    a.ntgt = p.num_targets;
    a.kc = static_cast<const float*>(p.k_cache);
    a.vc = static_cast<const float*>(p.v_cache);
    a.hoff = p.hist_offsets;
    a.ts = p.timestamps;
    a.hts = p.hist_timestamps;
    a.wpos = p.pos_bias;
    a.wtime = p.time_bias;
    a.npos = p.num_pos;
    a.ntime = p.num_time;
    a.row_stride = p.dense ? p.d : (int64_t)p.heads * p.d;
    a.head_stride = p.dense ? p.dense_len * p.d : p.d;
    a.wl = wl;
    a.num_seqs = p.num_seqs;
    a.heads = p.heads;
    a.score_scale = -p.alpha * LOG2E;
    a.out_scale = -LN2 / p.n;
    a.clk = p.clk;
    a.clk_id = p.clk_id;
    auto fn = wl.fused ? attn_fwd_mfma_f32<D, NWF, BKF, true> : attn_fwd_mfma_f32<D, NWF, BKF, false>;
    if (grid <= 0) {
        static int cached[2] = {0, 0};
        int& c = cached[wl.fused ? 1 : 0];
        if (!c) c = resident_grid(fn, NWF * 64);
        grid = c;
    }
    if (start)
        hipExtLaunchKernelGGL(fn, dim3(grid), dim3(NWF * 64), 0, stream, start, stop, 0, a);
    else
        hipLaunchKernelGGL(fn, dim3(grid), dim3(NWF * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

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

int q_tile_rows(Dtype dt, int d, bool single_block) {
    if (dt == Dtype::FP32) return TileF32<64, NWF, BKF>::BQ;
    if (single_block)
        return d == 64 ? Tile16<__bf16, 64, NW16, QBlocksFor<64, MASK_CACHED>::value,
                                KeyTile<64>::value, Prefetch<64>::value>::BQ
                       : Tile16<__bf16, 128, NW16, QBlocksFor<128, MASK_CACHED>::value,
                                KeyTile<128>::value, Prefetch<128>::value>::BQ;
    return d == 64 ? Tile16<__bf16, 64, NW16, QBlocks<64>::value, KeyTile<64>::value,
                            Prefetch<64>::value>::BQ
                   : Tile16<__bf16, 128, NW16, QBlocks<128>::value, KeyTile<128>::value,
                            Prefetch<128>::value>::BQ;
}

hipError_t launch_attention(const FwdParams& p, Dtype dt, WorkList wl, int grid,
                            hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    switch (dt) {
    case Dtype::BF16:
        return p.d == 64 ? launch16<__bf16, 64>(p, wl, grid, stream, start, stop)
                         : launch16<__bf16, 128>(p, wl, grid, stream, start, stop);
    case Dtype::FP16:
        return p.d == 64 ? launch16<_Float16, 64>(p, wl, grid, stream, start, stop)
                         : launch16<_Float16, 128>(p, wl, grid, stream, start, stop);
    case Dtype::FP32:
        return p.d == 64 ? launch_f32<64>(p, wl, grid, stream, start, stop)
                         : launch_f32<128>(p, wl, grid, stream, start, stop);
    }
    return hipErrorInvalidValue;
}

}  // namespace hstu
