// la_gdn_fwd_noalloc: the forward with its workspace in a fixed device array of the
// library, for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).  Everything else is la_gdn_fwd:
// the same checks, the same kernels, the same results bit for bit.
//
// The array `scratch` below is a file-scope __device__ variable: each GPU the library runs
// on holds its own copy (kScratchBytes) from the first launch until the process ends.  In
// host code its name is only a host-side stand-in, never a device address; its address on
// the current device comes from hipGetSymbolAddress, looked up once per device (with that
// device current) and kept, and only that address is passed on.  No call here allocates:
// no hipMalloc, no hipFree, no allocating library routine.  The kernels need nothing in
// the workspace to start at zero (every word they read was written earlier in the same
// call), so nothing is cleared.  Calls that overlap on one GPU share the array and race.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "la_gdn.h"
#include "la_gdn_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The array's address on the current device (looked up on the first call per device).
la_status scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return la::fail_message(LA_ERR_HIP, "la_gdn_fwd_noalloc: hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
        return la::fail_message(LA_ERR_UNSUPPORTED, "la_gdn_fwd_noalloc: device index beyond 63");
    std::lock_guard<std::mutex> g(g_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            char msg[256];
            std::snprintf(msg, sizeof msg, "la_gdn_fwd_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
                          hipGetErrorString(e));
            return la::fail_message(LA_ERR_HIP, msg);
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LA_OK;
}

}  // namespace

extern "C" la_status la_gdn_fwd_noalloc(const la_gdn_desc *desc, const void *q, const void *k, const void *v,
                                        const float *g, const float *beta, const int32_t *cu_seqlens,
                                        const float *initial_state, void *out, float *final_state, int l2norm,
                                        hipStream_t stream)
{
    const size_t need = la_gdn_workspace_bytes(desc, 0);
    if (need == 0) return la_gdn_fwd(desc, q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, l2norm,
                                     nullptr, 0, stream);   // the descriptor's own error
    if (need > kScratchBytes) {
        char msg[256];
        std::snprintf(msg, sizeof msg,
                      "la_gdn_fwd_noalloc: the problem needs %zu bytes of workspace, more than the library's "
                      "fixed %zu-byte scratch array; call la_gdn_fwd with a workspace instead",
                      need, kScratchBytes);
        return la::fail_message(LA_ERR_WORKSPACE_TOO_SMALL, msg);
    }
    void *ws = nullptr;
    const la_status st = scratch_address(&ws);
    if (st != LA_OK) return st;
    return la_gdn_fwd(desc, q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, l2norm, ws,
                      kScratchBytes, stream);
}
