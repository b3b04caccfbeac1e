// la_noalloc.hip -- la_fwd_noalloc: la_fwd with its workspace in a static
// device array, for callers that cannot allocate device memory.
//
// The workspace of la_fwd (the per-segment state records and their prefixes)
// lives in `scratch`, a file-scope device array of kScratchBytes that every
// device the library runs on holds until the process ends.  Host code never
// uses the array's name as an address (in host code it is a stand-in, not a
// device pointer): on its first call on a device, with that device current,
// the entry point looks the device address up with hipGetSymbolAddress and
// keeps it per device; kernels get that address, as la_fwd's kernels get the
// caller's workspace.  Nothing needs clearing: la_fwd writes every record it
// reads.  Calls that overlap in time on one device share the array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "linattn.h"

namespace la {
la_status api_fail(la_status st, const char *msg);   // la_api.hip: sets la_last_error
}

namespace {

constexpr size_t kScratchBytes = (size_t)LA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The device address of `scratch` on the current device (looked up once).
la_status scratch_here(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return la::api_fail(LA_ERR_HIP, "HIP: no current device");
    if (dev >= kMaxDevices) return la::api_fail(LA_ERR_UNSUPPORTED, "device ordinal beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return la::api_fail(LA_ERR_HIP, "HIP: the scratch array has no device address");
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LA_OK;
}

}  // namespace

extern "C" la_status la_fwd_noalloc(const void *q, const void *k, const void *v, void *out, int B,
                                    int H, int H_kv, int N, int D, int dtype, int causal,
                                    int phi, float eps, const float *cos_w, const float *sin_w,
                                    void *stream) {
    const size_t need = la_workspace_bytes(LA_OP_FWD, B, H, H_kv, N, D, dtype, causal,
                                           cos_w != nullptr);
    if (need == 0)   // arguments la_fwd rejects: let it say why
        return la_fwd(q, k, v, out, B, H, H_kv, N, D, dtype, causal, phi, eps, cos_w, sin_w,
                      nullptr, 0, stream);
    if (need > kScratchBytes)
        return la::api_fail(LA_ERR_INVALID,
                            "la_fwd_noalloc: these sizes need more workspace than the "
                            "LA_NOALLOC_SCRATCH_BYTES (40 MiB) the library holds; use la_fwd");
    if (stream != nullptr) {   // the stream's device must be the current one
        int cur = -1;
        hipDevice_t sdev = -1;
        if (hipGetDevice(&cur) != hipSuccess ||
            hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
            return la::api_fail(LA_ERR_HIP, "HIP: cannot tell the stream's device");
        if (sdev != cur)
            return la::api_fail(LA_ERR_INVALID,
                                "la_fwd_noalloc: the stream belongs to another device than the "
                                "current one");
    }
    void *ws = nullptr;
    const la_status st = scratch_here(&ws);
    if (st != LA_OK) return st;
    return la_fwd(q, k, v, out, B, H, H_kv, N, D, dtype, causal, phi, eps, cos_w, sin_w, ws,
                  kScratchBytes, stream);
}
