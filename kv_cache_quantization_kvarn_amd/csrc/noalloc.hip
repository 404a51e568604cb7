// kvarn_decode_attn_noalloc: kvarn_decode_attn with its split-K workspace in
// a fixed device array of this library instead of a caller-provided buffer,
// for callers that cannot allocate device memory.
//
// The array lives in every GPU the library runs on until the process ends.
// Its address on a device is looked up once (hipGetSymbolAddress, with that
// device current) and kept; host code never passes the array's own name to a
// kernel (on the host that name is a stand-in, not a device address).  All
// calls on one GPU share the array: calls that overlap on one GPU (on
// different streams, or from several threads) race on it and must be ordered
// by the caller.  The decode kernels overwrite every workspace byte they read,
// so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvarn.h"
#include "kvarn_internal.hpp"

namespace {

constexpr size_t kScratchBytes = KVARN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of the array (set-up on first use).
hipError_t scratch_ptr(int dev, void** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" kvarn_status kvarn_decode_attn_noalloc(const kvarn_layout* layout, const kvarn_cache* cache,
                                                  const kvarn_page_table* pages, const void* q, int32_t q_dtype,
                                                  int32_t num_q_heads, float sm_scale, float* out, void* stream) {
    if (!layout || !pages) return kvarn_decode_attn(layout, cache, pages, q, q_dtype, num_q_heads, sm_scale, out,
                                                    nullptr, 0, stream);  // the usual argument error
    const size_t need = kvarn_decode_workspace_bytes(layout, pages->batch, num_q_heads, pages->max_pages);
    if (need == 0)  // invalid layout or shape: the same status and message as kvarn_decode_attn
        return kvarn_decode_attn(layout, cache, pages, q, q_dtype, num_q_heads, sm_scale, out, nullptr, 0, stream);
    if (need > kScratchBytes) {
        return kvarn::set_error(KVARN_EWORKSPACE,
                                "decode workspace of %zu bytes exceeds the library's fixed %zu-byte array "
                                "(KVARN_NOALLOC_SCRATCH_BYTES); use kvarn_decode_attn with a workspace",
                                need, kScratchBytes);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
    void* ws = nullptr;
    if (e == hipSuccess) e = scratch_ptr(dev, &ws);
    if (e != hipSuccess) {
        return kvarn::set_error(KVARN_EHIP, "no address for the fixed workspace array on device %d: %s", dev,
                                hipGetErrorString(e));
    }
    return kvarn_decode_attn(layout, cache, pages, q, q_dtype, num_q_heads, sm_scale, out, ws, kScratchBytes, stream);
}
