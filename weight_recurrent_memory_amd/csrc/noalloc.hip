// la_forward_noalloc: la_forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, hosts that
// forbid allocation).  Its workspace is a file-scope device array, one copy
// per GPU the library runs on, held until the process ends; the call itself
// allocates and frees nothing.
//
// Host code never uses the array's name as an address (on the host it is a
// stand-in, not a device pointer): hipGetSymbolAddress gives each device's
// copy, once per device with that device current, and that pointer is what
// the kernels receive.  Every call on one GPU shares its copy, so calls that
// may overlap on one GPU race.  Nothing in the array has to start at zero:
// the look-back flags carry the tag of the call that wrote them.
#include <stdio.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "api_internal.hpp"
#include "linattn.h"

namespace {

constexpr size_t kScratchBytes = (size_t)LA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call made
// with that device current.
la_status scratch_for_current_device(const char* fn, void** out) {
    char msg[256];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        snprintf(msg, sizeof(msg), "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
        return la_api::set_error(LA_ERR_HIP, msg);
    }
    if (dev < 0 || dev >= kMaxDevices) {
        snprintf(msg, sizeof(msg), "%s: device %d beyond the %d this call keeps scratch for", fn, dev, kMaxDevices);
        return la_api::set_error(LA_ERR_UNSUPPORTED, msg);
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            snprintf(msg, sizeof(msg), "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                     hipGetErrorString(e));
            return la_api::set_error(LA_ERR_HIP, msg);
        }
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return LA_OK;
}

}  // namespace

extern "C" la_status la_forward_noalloc(const void* q, const void* k, const void* v, const float* S0,
                                        const float* z0, void* o, float* S_out, float* z_out, int B, int H, int T,
                                        int dk, int dv, int dtype, float eps, int chunk, void* stream) {
    const char* fn = "la_forward_noalloc";
    // the size the workspace would have; beyond the fixed scratch, refuse
    // before touching the device (0 = invalid sizes, which la_forward_ws reports)
    const size_t need = la_api::la_forward_ws_bytes(fn, B, H, T, dk, dv, chunk);
    if (need > kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof(msg), "%s: these sizes need %zu bytes of workspace; the fixed scratch holds %zu", fn,
                 need, kScratchBytes);
        return la_api::set_error(LA_ERR_UNSUPPORTED, msg);
    }
    void* ws = nullptr;
    if (need > 0) {
        const la_status st = scratch_for_current_device(fn, &ws);
        if (st != LA_OK) return st;
    }
    return la_api::la_forward_ws(fn, q, k, v, S0, z0, o, S_out, z_out, B, H, T, dk, dv, dtype, eps, chunk, ws,
                                 ws ? kScratchBytes : 0, stream);
}
