// Device helpers shared by the forward and backward kernels (gfx950).
#ifndef HSTU_DEVICE_COMMON_H_
#define HSTU_DEVICE_COMMON_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// ---------------------------------------------------------------------------
// Buffer resources.  Every load and store goes through a raw buffer whose
// range ends at the current sequence's last token: a load past it returns
// zero and a store past it is dropped, so tile tails need no predicates and
// nothing outside the sequence is ever touched.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int RSRC_WORD3 = 0x00020000;  // gfx9 raw buffer, 32-bit data format

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations and does not wait on the other counters (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
#define VMCNT_LE(n) ((((n) & 15) | ((((n) >> 4) & 3) << 14)) | (7 << 4) | (15 << 8))

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, RSRC_WORD3);
}

// Same, for a byte count already known to fit in 32 bits (no 64-bit compares).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, max(bytes, 0),
                                             RSRC_WORD3);
}

// Loads from a raw buffer straight into LDS (buffer_load ... lds): lane l's
// bytes land at lds_base + size * l (lds_base wave-uniform, set in M0);
// out-of-range lanes write zero.
//
// They are issued through inline assembly so that the compiler does not track
// them.  The compiler cannot tell which LDS bytes a load still in flight will
// write, so after a tracked one it waits for every outstanding load (s_waitcnt
// vmcnt(0)) before any LDS read: a kernel that reads one tile while the next
// ones stream in would then wait for those next tiles first.  Every caller
// therefore orders its LDS reads itself, with explicit vmcnt waits (and
// barriers between waves) before it reads a staged tile.  The instructions
// write no VGPR; M0 is set inside, with the wait state an M0 write needs
// before an LDS DMA, and given back its value afterwards (the load reads M0
// when it issues).  The host pass, which compiles kernel bodies into launch
// stubs but never runs them, gets empty bodies.
#define HSTU_LDS_DMA(op)                                                                   \
    typedef __attribute__((address_space(3))) unsigned char lds_u8;                          \
    const unsigned m0 = (unsigned)(uintptr_t)(lds_u8*)lds_base;                              \
    unsigned saved;                                                                          \
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t" op                    \
                 " %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"                                   \
                 : "=&s"(saved)                                                              \
                 : "s"(m0), "v"(voffset), "s"(r)                                             \
                 : "memory")

__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char* lds_base,
                                              int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    HSTU_LDS_DMA("buffer_load_dwordx4");
#else
    (void)r;
    (void)lds_base;
    (void)voffset;
#endif
}

__device__ __forceinline__ void load4_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char* lds_base,
                                             int voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    HSTU_LDS_DMA("buffer_load_dword");
#else
    (void)r;
    (void)lds_base;
    (void)voffset;
#endif
}
#undef HSTU_LDS_DMA

// LDS transposing read of four 16-bit values (gfx950 ds_read_b64_tr_b16).
// Within each group of 16 lanes, lane i receives element (i % 4) of the
// 8 bytes addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12 of its group.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// K: 16 lanes of a 16-byte read hit 16 consecutive rows at one chunk.
template <int CHUNKS>
__device__ __forceinline__ int kswz(int r) {
    if constexpr (CHUNKS == 8) return (r >> 1) & 7;
    else return (2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1)) & (CHUNKS - 1);
}
// V: a 16-lane transposing read hits 4 consecutive rows at two adjacent chunks.
template <int CHUNKS>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (CHUNKS == 8) return (2 * (r & 3) + ((r >> 2) & 1)) & 7;
    else return (2 * (r & 3) + ((r >> 2) & 1) + 8 * ((r >> 3) & 1)) & (CHUNKS - 1);
}

}  // namespace
}  // namespace hstu

#endif  // HSTU_DEVICE_COMMON_H_
