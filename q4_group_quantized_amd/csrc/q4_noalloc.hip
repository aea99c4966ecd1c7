// q4_noalloc.hip -- q4_gemv_topk for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): the same kernels as q4_gemv_topk, with their scratch
// (per-workgroup candidate lists, and the logits at m > 1) in a fixed buffer
// that the library itself holds on every device it runs on.
//
// `scratch` below is a file-scope device array.  In host code its name is a
// host-side stand-in, not a device address, so it is never passed to a
// kernel or a copy: the first call on a device looks up that device's copy
// with hipGetSymbolAddress (with the device current) and every later call
// on that device uses the address found then.  Each device holds its own
// copy at its own address.
//
// Every call on one device shares that device's buffer.  Nothing in it needs
// to start at zero: every list and every logit is written before it is read
// within the same call.  Calls that overlap in time on one device (other
// streams, other host threads) race on it and must be serialised by the
// caller.
#include "q4.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = (size_t)Q4_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};    // device address of `scratch`, per device

// This device's copy of `scratch`, looked up once per device while it is
// current.  No allocation: the array is part of the loaded code object.
hipError_t scratch_address(int device, void** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace

extern "C" q4_status q4_gemv_topk_noalloc(const uint16_t* x, const uint8_t* packed,
                                          const uint16_t* scales, int64_t m, int64_t n,
                                          int64_t k, int32_t topk, float* values,
                                          int32_t* rows, void* stream) {
    // Every argument check of q4_gemv_topk, in its order: with no workspace
    // it launches nothing, and reports Q4_ERR_WORKSPACE only when all the
    // other arguments are valid.
    const q4_status st =
        q4_gemv_topk(x, packed, scales, m, n, k, topk, values, rows, nullptr, 0, stream);
    if (st != Q4_ERR_WORKSPACE) return st;
    const size_t need = q4_gemv_topk_workspace_size(m, n, k);
    if (need == 0) return Q4_ERR_DEVICE;
    if (need > kScratchBytes) return Q4_ERR_TOO_LARGE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q4_ERR_DEVICE;
    void* ws = nullptr;
    if (scratch_address(dev, &ws) != hipSuccess) return Q4_ERR_LAUNCH;
    return q4_gemv_topk(x, packed, scales, m, n, k, topk, values, rows, ws, kScratchBytes,
                        stream);
}
