// The allocation-free forward entry point: the work list lives in a file-scope
// device array instead of the library's per-stream scratch area.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "hstu.h"
#include "internal.h"

// One copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in: the device address comes from
// hipGetSymbolAddress, per device, and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[HSTU_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_mu;
std::map<int, void*> g_addr;   // device -> address of that device's `scratch`

// The address of `scratch` on the current device `dev` (looked up once per
// device, with that device current).
hstu_status_t scratch_address(int dev, void** out) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_addr.find(dev);
    if (it == g_addr.end()) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hstu::hip_error_status(e);
        if (!p) return HSTU_ERR_HIP;
        it = g_addr.emplace(dev, p).first;
    }
    *out = it->second;
    return HSTU_OK;
}

}  // namespace

extern "C" hstu_status_t hstu_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                                               const int32_t* seq_offsets, int32_t num_seqs,
                                               int32_t heads, int32_t d, float alpha, float n,
                                               void* out, hipStream_t stream,
                                               hstu_dtype_t dtype) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hstu::hip_error_status(e);
    void* area = nullptr;
    const hstu_status_t st = scratch_address(dev, &area);
    if (st != HSTU_OK) return st;
    return hstu::attn_fwd_fixed_area(q, k, v, seq_offsets, num_seqs, heads, d, alpha, n, out,
                                     stream, (int)dtype, area, HSTU_NOALLOC_SCRATCH_BYTES);
}
