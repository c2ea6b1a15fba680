// gdn_noalloc.hip -- gdn_fwd_step_noalloc: gdn_fwd_step with its scratch
// memory in a static device array instead of a caller-supplied workspace, for
// callers that cannot allocate (code under graph capture, serving loops,
// harnesses that forbid hipMalloc).
//
// The array `scratch` below is a device symbol: host code never passes its
// name to a kernel or a copy.  At the first call on a device, with that device
// current, hipGetSymbolAddress gives the array's address on that device; it is
// kept per device and used as the workspace from then on.  Every call on a
// device shares that device's array, which keeps the last call's contents:
// calls that overlap on one device (different streams, different host
// threads) race on it.  No kernel of the step reads workspace bytes it has not
// written in the same call, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdio.h>

#include "gdn.h"
#include "gdn_kernels.h"

namespace {

constexpr size_t kScratchBytes = GDN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Address of this device's scratch array (resolved once per device).
hipError_t scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int gdn_fwd_step_noalloc(const void* q, const void* k, const void* v, const void* alpha, const void* beta,
                         const float* state_in, void* out, float* state_out,
                         int B, int H, int T, int dk, int dv, const gdn_opts* opts) {
    gdn_opts o;
    if (opts) o = *opts; else gdn_default_opts(&o);
    o.workspace = nullptr;
    o.workspace_bytes = 0;
    const size_t need = gdn_workspace_bytes(B, H, T, dk, dv, 0, &o);
    char msg[256];
    if (need > kScratchBytes) {
        snprintf(msg, sizeof(msg),
                 "gdn_fwd_step_noalloc: this shape needs %zu bytes of scratch, above the static %zu",
                 need, kScratchBytes);
        return gdn::api_fail(GDN_ERR_UNSUPPORTED, msg);
    }
    if (need > 0) {
        void* p = nullptr;
        const hipError_t e = scratch_ptr(&p);
        if (e != hipSuccess) {
            snprintf(msg, sizeof(msg), "gdn_fwd_step_noalloc: hipGetSymbolAddress failed: %s",
                     hipGetErrorString(e));
            return gdn::api_fail(GDN_ERR_HIP, msg);
        }
        o.workspace = p;
        o.workspace_bytes = kScratchBytes;
    }
    return gdn_fwd_step(q, k, v, alpha, beta, state_in, out, state_out, B, H, T, dk, dv, &o);
}

}  // extern "C"
