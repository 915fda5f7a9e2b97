// moe_layer_forward_noalloc: the whole layer with its workspace in a fixed
// device array of the library, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Declared and documented in moe.h.
//
// `scratch` is a file-scope device array: in host code its name is only a
// stand-in for the symbol, never a device address.  On the first call on a
// device (with that device current) hipGetSymbolAddress gives this device's
// copy of the array; the address is kept per device and is what the kernels
// receive, exactly as they receive the caller's workspace in
// moe_layer_forward.  Nothing else is allocated.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "common.h"
#include "devinfo.h"
#include "moe.h"

namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;

int fail(char* err, size_t len, int code, const char* fmt, ...) {
    if (err && len > 0) {
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(err, len, fmt, ap);
        va_end(ap);
    }
    return code;
}

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of this device's `scratch`, looked up once per device.
std::atomic<uintptr_t> g_scratch[moe::kMaxDevices];

int scratch_address(void** out, char* err, size_t err_len) {
    const int dev = moe::current_device();
    if (dev >= moe::kMaxDevices)
        return fail(err, err_len, MOE_EUNSUPPORTED, "device %d is beyond the %d this build tracks", dev,
                    moe::kMaxDevices);
    uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        void* q = nullptr;
        const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !q)
            return fail(err, err_len, MOE_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        p = (uintptr_t)q;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = (void*)p;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_layer_forward_noalloc(const moe_shape* shape, const void* x, const float* w_router, const float* b_router,
                              const moe_weights* w, const void* residual, void* y, int32_t* counts_out,
                              int32_t* topk_idx_out, void* stream, char* err, size_t err_len) {
    // shape errors come back from moe_layer_forward with their own message;
    // a valid shape must fit the fixed array
    const size_t need = moe_workspace_bytes(shape);
    if (need > kScratchBytes)
        return fail(err, err_len, MOE_ENOMEM,
                    "this shape needs %zu bytes of workspace; the fixed device array holds %zu (use "
                    "moe_layer_forward with a caller workspace)",
                    need, kScratchBytes);
    if (need == 0)
        return moe_layer_forward(shape, x, w_router, b_router, w, residual, y, counts_out, topk_idx_out, nullptr,
                                 0, stream, err, err_len);
    void* ws = nullptr;
    const int rc = scratch_address(&ws, err, err_len);
    if (rc) return rc;
    return moe_layer_forward(shape, x, w_router, b_router, w, residual, y, counts_out, topk_idx_out, ws,
                             kScratchBytes, stream, err, err_len);
}

}  // extern "C"
