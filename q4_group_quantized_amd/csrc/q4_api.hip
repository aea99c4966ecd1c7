// q4_api.hip -- the C ABI declared in include/q4.h: argument validation,
// status mapping and kernel dispatch.  Every check here runs on the host,
// synchronously, before anything is enqueued; the kernels themselves assume
// validated arguments.
#include "q4.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "q4_launch.hpp"

namespace q4 {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
DeviceInfo g_dev_info[kMaxDevices];
bool g_dev_ready[kMaxDevices] = {};
bool g_dev_ok[kMaxDevices] = {};

// Fills the cache entry for `device`; returns false when it is not a gfx950.
bool probe_device(int device) {
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (!g_dev_ready[device]) {
        hipDeviceProp_t prop;
        bool ok = hipGetDeviceProperties(&prop, device) == hipSuccess;
        if (ok) {
            ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            g_dev_info[device].cu_count = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1;
        }
        g_dev_ok[device] = ok;
        g_dev_ready[device] = true;
    }
    return g_dev_ok[device];
}
}  // namespace

const DeviceInfo& device_info(int device) {
    probe_device(device);
    return g_dev_info[device];
}

bool device_usable(int device) { return probe_device(device); }

hipError_t allow_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < kMaxDevices) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

}  // namespace q4

namespace {

constexpr int64_t kMaxN = 0x7FFFFFFFLL;
constexpr int64_t kMaxK = 1LL << 24;
constexpr int64_t kMaxElems = 1LL << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

q4_status check_nk(int64_t n, int64_t k) {
    if (n < 1 || n > kMaxN || k < 32 || k > kMaxK || (k % 32) != 0) return Q4_ERR_SHAPE;
    if (n > kMaxElems / k) return Q4_ERR_SHAPE;
    return Q4_OK;
}

q4_status device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return Q4_ERR_DEVICE;
    return q4::device_usable(dev) ? Q4_OK : Q4_ERR_DEVICE;
}

q4_status map_launch(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_LAUNCH; }

q4_status check_product(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                        const float* y, int64_t m, int64_t n, int64_t k, int64_t m_max) {
    if (!x || !packed || !scales || !y) return Q4_ERR_NULL;
    q4_status st = check_nk(n, k);
    if (st != Q4_OK) return st;
    if (m < 1 || m > m_max) return Q4_ERR_SHAPE;
    if (m > kMaxElems / k || m > kMaxElems / n) return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    return Q4_OK;
}

}  // namespace

extern "C" {

int q4_abi_version(void) { return Q4_ABI_VERSION; }

const char* q4_status_str(q4_status status) {
    switch (status) {
        case Q4_OK: return "ok";
        case Q4_ERR_NULL: return "null pointer argument";
        case Q4_ERR_SHAPE: return "shape out of range (need n>=1, k>=32, k%32==0, m and count in range)";
        case Q4_ERR_ALIGN: return "misaligned pointer (x, packed, w: 16 B; scales: 2 B; y: 4 B)";
        case Q4_ERR_LAUNCH: return "kernel launch failed";
        case Q4_ERR_DEVICE: return "current device is not a usable gfx950";
        case Q4_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case Q4_ERR_TOO_LARGE: return "problem needs more scratch than the built-in buffer holds";
    }
    return "unknown status";
}

q4_status q4_quantize(const float* w, uint8_t* packed, uint16_t* scales, int64_t n, int64_t k,
                      void* stream) {
    if (!w || !packed || !scales) return Q4_ERR_NULL;
    q4_status st = check_nk(n, k);
    if (st != Q4_OK) return st;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return Q4_ERR_ALIGN;
    if ((st = device_ok()) != Q4_OK) return st;
    return map_launch(q4::launch_quantize(w, packed, scales, n, k,
                                          static_cast<hipStream_t>(stream)));
}

q4_status q4_gemv(const uint16_t* x, const uint8_t* packed, const uint16_t* scales, float* y,
                  int64_t m, int64_t n, int64_t k, void* stream) {
    q4_status st = check_product(x, packed, scales, y, m, n, k, 8);
    if (st != Q4_OK) return st;
    if ((st = device_ok()) != Q4_OK) return st;
    return map_launch(q4::launch_gemv(x, packed, scales, y, m, n, k,
                                      static_cast<hipStream_t>(stream)));
}

q4_status check_multi(const uint16_t* x, int64_t m, int64_t k, int32_t count,
                      const uint8_t* const* packed, const uint16_t* const* scales,
                      float* const* y, const int64_t* n, int64_t m_max) {
    if (!packed || !scales || !y || !n) return Q4_ERR_NULL;
    if (count < 1 || count > Q4_MULTI_MAX) return Q4_ERR_SHAPE;
    for (int32_t i = 0; i < count; ++i) {
        const q4_status st = check_product(x, packed[i], scales[i], y[i], m, n[i], k, m_max);
        if (st != Q4_OK) return st;
    }
    return device_ok();
}

q4_status q4_gemv_multi(const uint16_t* x, int64_t m, int64_t k, int32_t count,
                        const uint8_t* const* packed, const uint16_t* const* scales,
                        float* const* y, const int64_t* n, void* stream) {
    const q4_status st = check_multi(x, m, k, count, packed, scales, y, n, 8);
    if (st != Q4_OK) return st;
    return map_launch(q4::launch_gemv_multi(x, m, k, count, packed, scales, y, n,
                                            static_cast<hipStream_t>(stream)));
}

q4_status q4_gemm_multi(const uint16_t* x, int64_t m, int64_t k, int32_t count,
                        const uint8_t* const* packed, const uint16_t* const* scales,
                        float* const* y, const int64_t* n, void* stream) {
    const q4_status st = check_multi(x, m, k, count, packed, scales, y, n, kMaxN);
    if (st != Q4_OK) return st;
    return map_launch(q4::launch_gemm_multi(x, m, k, count, packed, scales, y, n,
                                            static_cast<hipStream_t>(stream)));
}

q4_status q4_gemv_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m, int64_t n,
                      int64_t k, void* stream) {
    if (!x || !w || !y) return Q4_ERR_NULL;
    q4_status st = check_nk(n, k);
    if (st != Q4_OK) return st;
    if (m < 1 || m > 8) return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    if ((st = device_ok()) != Q4_OK) return st;
    return map_launch(q4::launch_gemv_f16(x, w, y, m, n, k, static_cast<hipStream_t>(stream)));
}

q4_status q4_gemm_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m, int64_t n,
                      int64_t k, void* stream) {
    if (!x || !w || !y) return Q4_ERR_NULL;
    q4_status st = check_nk(n, k);
    if (st != Q4_OK) return st;
    if (m < 1 || m > kMaxN || m > kMaxElems / k || m > kMaxElems / n) return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 4)) return Q4_ERR_ALIGN;
    if ((st = device_ok()) != Q4_OK) return st;
    return map_launch(q4::launch_gemm_f16(x, w, y, m, n, k, static_cast<hipStream_t>(stream)));
}

size_t q4_gemv_topk_workspace_size(int64_t m, int64_t n, int64_t k) {
    if (check_nk(n, k) != Q4_OK || m < 1 || m > 8) return 0;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64 || !q4::device_usable(dev))
        return 0;
    return q4::gemv_topk_workspace(m, n, k, q4::device_info(dev).cu_count);
}

q4_status q4_gemv_topk(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                       int64_t m, int64_t n, int64_t k, int32_t topk, float* values,
                       int32_t* rows, void* workspace, size_t workspace_bytes, void* stream) {
    if (!x || !packed || !scales || !values || !rows) return Q4_ERR_NULL;
    q4_status st = check_nk(n, k);
    if (st != Q4_OK) return st;
    if (m < 1 || m > 8 || topk < 1 || topk > Q4_TOPK_MAX || topk > n || n > 0x7FFFFFFE)
        return Q4_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(values, 4) ||
        !aligned(rows, 4))
        return Q4_ERR_ALIGN;
    if ((st = device_ok()) != Q4_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return Q4_ERR_DEVICE;
    const size_t need = q4::gemv_topk_workspace(m, n, k, q4::device_info(dev).cu_count);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return Q4_ERR_WORKSPACE;
    return map_launch(q4::launch_gemv_topk(x, packed, scales, m, n, k, topk, values, rows,
                                           workspace, static_cast<hipStream_t>(stream)));
}

q4_status q4_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* scales, float* y,
                  int64_t m, int64_t n, int64_t k, void* stream) {
    q4_status st = check_product(x, packed, scales, y, m, n, k, kMaxN);
    if (st != Q4_OK) return st;
    if ((st = device_ok()) != Q4_OK) return st;
    return map_launch(q4::launch_gemm(x, packed, scales, y, m, n, k,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
