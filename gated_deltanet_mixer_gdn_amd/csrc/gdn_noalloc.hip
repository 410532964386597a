// gdn_noalloc.hip - gdn_project_bf16_noalloc: the projection of gdn_project_bf16 for
// callers that cannot allocate device memory or hand in a workspace (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).  The k-split
// launches of the projection need a scratch buffer for their partial blocks; here it is
// a fixed array in the library's own device memory, one copy per GPU, held until the
// process ends.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "gdn.h"
#include "gdn_gemm.h"

namespace {

constexpr size_t kScratchBytes = GDN_PROJECT_SCRATCH_BYTES;

// The partial blocks of a k-split projection.  Its name in host code is a host-side
// stand-in, not a device address: host code only ever uses the per-device address
// hipGetSymbolAddress returns for it (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of this device's copy of `scratch`, looked up once per device with that
// device current (each GPU holds the array at an address of its own).
int scratch_ptr(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    char msg[256];
    if (e != hipSuccess) {
        std::snprintf(msg, sizeof msg, "hipGetDevice: %s", hipGetErrorString(e));
        return gdn::set_last_error(GDN_ERR_HIP, fn, msg);
    }
    if (dev < 0 || dev >= kMaxDevices) {
        std::snprintf(msg, sizeof msg, "device %d: the scratch buffer serves devices 0 to %d", dev, kMaxDevices - 1);
        return gdn::set_last_error(GDN_ERR_UNSUPPORTED, fn, msg);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void) hipGetLastError();
            std::snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                          hipGetErrorString(e));
            return gdn::set_last_error(GDN_ERR_HIP, fn, msg);
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" int gdn_project_bf16_noalloc(const uint16_t* xs, const uint16_t* wp, int64_t rows, int32_t k, int32_t n,
                                        float* out, void* stream) {
    const char* fn = "gdn_project_bf16_noalloc";
    const int64_t need = gdn_project_workspace_bytes(rows, k, n);
    // a bad shape, or one that needs no workspace: the plain call reports or does it
    if (need <= 0) {
        const int rc = gdn_project_bf16(xs, wp, rows, k, n, out, nullptr, 0, stream);
        if (rc != GDN_OK) {
            char msg[512];
            std::snprintf(msg, sizeof msg, "%s", gdn_last_error());
            return gdn::set_last_error(rc, fn, msg);
        }
        return rc;
    }
    if ((uint64_t) need > kScratchBytes) {
        char msg[256];
        std::snprintf(msg, sizeof msg,
                      "rows=%lld k=%d n=%d needs %lld bytes of workspace, more than the %zu of the library's "
                      "scratch buffer (gdn_project_bf16 takes a workspace of the caller's)",
                      (long long) rows, k, n, (long long) need, kScratchBytes);
        return gdn::set_last_error(GDN_ERR_ARG, fn, msg);
    }
    void* ptr = nullptr;
    if (int rc = scratch_ptr(fn, &ptr)) return rc;
    const int rc = gdn_project_bf16(xs, wp, rows, k, n, out, ptr, (int64_t) kScratchBytes, stream);
    if (rc != GDN_OK) {
        char msg[512];
        std::snprintf(msg, sizeof msg, "%s", gdn_last_error());
        return gdn::set_last_error(rc, fn, msg);
    }
    return rc;
}
