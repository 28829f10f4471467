// fwt_ablation_execute_static: the ablations that need a workspace, run on
// scratch memory the library holds in a static device array, for callers
// that cannot allocate device memory themselves.
//
// The array lives in this code object.  The runtime places one copy on each
// device the library runs on, and that copy lasts until the process ends.
// Host code must never use the array's name as a device address.  The
// address of the current device's copy is looked up once per device with
// hipGetSymbolAddress, kept per device, and passed to the kernels like any
// caller workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fwt.h"
#include "fwt_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[FWT_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on
// the first call on that device.
int scratch_ptr(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return qse::hip_status(e);
    if (dev < 0 || dev >= kMaxDevices)
        return FWT_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return qse::hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
        }
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return FWT_OK;
}

}  // namespace

extern "C" int fwt_ablation_execute_static(int kind, int64_t batch, int n, fwt_dtype dtype,
                                           void* re, void* im, int normalize, hipStream_t stream)
{
    if (kind < FWT_ABLATION_STAGEWISE || kind > FWT_ABLATION_MFMA_TRANSPOSE || batch < 0 ||
        n < 0 || n > FWT_MAX_N || (dtype != FWT_F32 && dtype != FWT_F64))
        return FWT_EINVAL;
    const size_t need = qse::ablation_workspace_size(kind, batch, n, (int)dtype, im ? 1 : 0);
    if (need > (size_t)FWT_STATIC_SCRATCH_BYTES)
        return FWT_ESCRATCH;
    // Every argument check (the device-memory range queries included) runs
    // before the scratch lookup and before anything is enqueued.
    int rc = qse::ablation_validate(kind, batch, n, (int)dtype, re, im);
    if (rc != FWT_OK || batch == 0)
        return rc;
    void* ws = nullptr;
    if (need) {
        rc = scratch_ptr(&ws);
        if (rc != FWT_OK)
            return rc;
    }
    return qse::ablation_run(kind, batch, n, (int)dtype, re, im, normalize, ws,
                             need ? (size_t)FWT_STATIC_SCRATCH_BYTES : 0, true, stream);
}
