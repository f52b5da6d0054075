// Allocation-free decode entry point: moe_forward_decode with its workspace
// in a fixed device array of this library instead of a caller buffer, for
// callers that cannot allocate device memory (code under graph capture,
// serving loops that forbid allocation). Declaration and contract in
// include/moe_mxfp4.h.
//
// The array is a file-scope __device__ variable, so every GPU the library runs
// on holds its own copy from module load until the process ends. In host code
// its name is only a stand-in: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_status.hpp"
#include "moe_mxfp4.h"

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void *g_scratch[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (looked up on first use).
int scratch_ptr(void **out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moe::host_fail(MOE_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
        return moe::host_fail(MOE_ERR_UNSUPPORTED, "device index outside [0, 64)");
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (s != hipSuccess || !p)
            return moe::host_fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) failed");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_decode_noalloc(const moe_shape *s, const void *hidden,
                                          const float *norm_w, const float *router_w,
                                          const float *router_b, const moe_routing *routing,
                                          const uint8_t *experts, const uint8_t *shared,
                                          float *out, const moe_route_out *route_out,
                                          hipStream_t stream) {
    // the size check comes first and touches no device
    const size_t need = moe_workspace_bytes(s);
    if (need == 0) return MOE_ERR_INVALID_ARG;  // moe_workspace_bytes left the message
    if (need > kScratchBytes)
        return moe::host_fail(MOE_ERR_UNSUPPORTED,
                              "shape needs more workspace than the library's fixed "
                              "MOE_NOALLOC_SCRATCH_BYTES; use moe_forward_decode with a "
                              "caller workspace");
    if (s->T == 0) return moe_forward_decode(s, hidden, norm_w, router_w, router_b, routing,
                                             experts, shared, out, route_out, nullptr, 0, stream);
    void *ws = nullptr;
    const int rc = scratch_ptr(&ws);
    if (rc != MOE_OK) return rc;
    return moe_forward_decode(s, hidden, norm_w, router_w, router_b, routing, experts, shared,
                              out, route_out, ws, kScratchBytes, stream);
}
