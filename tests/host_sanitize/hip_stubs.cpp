// Stand-ins for the HIP runtime and for the kernel launchers, so that the host layer
// (la_gdn_api.cpp) can be built for the CPU alone under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Nothing here touches a device: a "launch" records the
// problem description it was given, events are counters, and copies from the
// "device" are plain memcpy from host buffers that stand in for device memory.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "la_gdn.h"
#include "la_gdn_internal.h"
#include "stub_record.h"

StubRecord g_stub;

namespace la {

hipError_t run_pipeline(const Prob &p, const Ws &w, bool summary, hipStream_t, const LaunchHook *hook)
{
    g_stub.pipeline_calls += 1;
    g_stub.last = p;
    g_stub.last_summary = summary;
    g_stub.last_ws = w;
    if (hook) {
        hook->before(LA_KERNEL_INTRA, nullptr, hook->ctx);
        hook->after(LA_KERNEL_INTRA, nullptr, hook->ctx);
    }
    return hipSuccess;
}

hipError_t convert_cu64(const int64_t *, int32_t *, int, hipStream_t)
{
    g_stub.cu64_calls += 1;
    return hipSuccess;
}

hipError_t run_summary_bwd(const Prob &p, const Ws &, const __bf16 *, const float *, float *, hipStream_t,
                           const LaunchHook *)
{
    g_stub.sbwd_calls += 1;
    g_stub.last = p;
    return hipSuccess;
}

hipError_t run_backward(const Prob &p, const Ws &w, const BwdArgs &, hipStream_t, const LaunchHook *)
{
    g_stub.bwd_calls += 1;
    g_stub.last = p;
    g_stub.last_ws = w;
    return hipSuccess;
}

}  // namespace la

extern "C" {

hipError_t hipGetDevice(int *d)
{
    *d = 0;
    return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t, int)
{
    *v = 256;
    return hipSuccess;
}

hipError_t hipEventCreate(hipEvent_t *e)
{
    static uintptr_t next = 0x1000;
    *e = reinterpret_cast<hipEvent_t>(next);
    next += 0x10;
    return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }

hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t)
{
    *ms = 0.5f;
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t)
{
    std::memcpy(dst, src, n);
    return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

const char *hipGetErrorString(hipError_t) { return "stub"; }

}  // extern "C"
