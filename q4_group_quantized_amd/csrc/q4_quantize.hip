// q4_quantize.hip -- symmetric 4-bit group quantization on gfx950.
//
// Method: QORA-4B forum article (section on quantization and memory
// management) and QORA-LLM-0.8B model card ("Weight Format"): 4-bit symmetric
// quantization in groups of 32 input elements.  Bit-level rules (scale =
// binary16(max|w| / 7), level = clamp(rne(w / scale), -8, 7), level 0 for a
// zero scale, code = level + 8 with the even element in the low nibble) are
// the ones the public header q4.h states; the result is unique, so this kernel
// must agree bit for bit with any other correct implementation.
//
// Mapping: 8 lanes per group, each lane owns 4 consecutive fp32 weights (one
// 16-byte load), so a wave reads 8 groups = 1 KiB of contiguous weights per
// load.  The group maximum is reduced over the 8 lanes with DPP-class lane
// exchanges; every lane then derives the same scale and quantizes its four
// weights.  Stores: 2 packed bytes per lane (128 contiguous bytes per wave)
// and one scale per group.
//
// Numerics: fp32 division is IEEE correctly rounded (hipcc default; this code
// must never be built with fast-math or approximate-division flags), fp32 and
// fp16 denormals are kept, rintf is round-half-to-even, and the fp32 -> fp16
// conversion rounds to nearest even.
#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kLanesPerGroup = 8;
constexpr int kGroupsPerBlock = kQuantThreads / kLanesPerGroup;

__device__ __forceinline__ int level_of(float w, float s) {
    float v = rintf(w / s);
    v = fminf(fmaxf(v, -8.0f), 7.0f);
    return s == 0.0f ? 0 : (int)v;
}

__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(
    const float* __restrict__ w, uint8_t* __restrict__ packed,
    uint16_t* __restrict__ scales, int64_t ngroups) {
    const int sub = threadIdx.x & (kLanesPerGroup - 1);
    const int64_t stride = (int64_t)gridDim.x * kGroupsPerBlock;
    // The loop bound is uniform per block so that all lanes of a group take
    // part in the lane exchange together.
    for (int64_t base = (int64_t)blockIdx.x * kGroupsPerBlock; base < ngroups;
         base += stride) {
        const int64_t g = base + (threadIdx.x / kLanesPerGroup);
        const bool live = g < ngroups;
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        if (live)
            v = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4_t*>(w + g * 32 + sub * 4));
        float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])),
                           fmaxf(fabsf(v[2]), fabsf(v[3])));
        amax = fmaxf(amax, __shfl_xor(amax, 1, kLanesPerGroup));
        amax = fmaxf(amax, __shfl_xor(amax, 2, kLanesPerGroup));
        amax = fmaxf(amax, __shfl_xor(amax, 4, kLanesPerGroup));

        const float ratio = amax / 7.0f;                    // IEEE fp32 division
        const _Float16 s16 = (_Float16)ratio;               // round to nearest even
        const float s = (float)s16;

        const int q0 = level_of(v[0], s) + 8;
        const int q1 = level_of(v[1], s) + 8;
        const int q2 = level_of(v[2], s) + 8;
        const int q3 = level_of(v[3], s) + 8;
        const uint16_t two_bytes =
            (uint16_t)((q0 | (q1 << 4)) | ((q2 | (q3 << 4)) << 8));
        if (live) {
            reinterpret_cast<uint16_t*>(packed + g * 16)[sub] = two_bytes;
            if (sub == 0)
                scales[g] = __builtin_bit_cast(uint16_t, s16);
        }
    }
}

}  // namespace

hipError_t launch_quantize(const float* w, uint8_t* packed, uint16_t* scales,
                           int64_t n, int64_t k, hipStream_t stream) {
    const int64_t ngroups = n * (k / 32);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const int64_t want = (ngroups + kGroupsPerBlock - 1) / kGroupsPerBlock;
    const int64_t cap = (int64_t)device_info(dev).cu_count * 16;
    const int blocks = (int)(want < cap ? want : cap);
    hipLaunchKernelGGL(quantize_kernel, dim3(blocks), dim3(kQuantThreads), 0,
                       stream, w, packed, scales, ngroups);
    return hipGetLastError();
}

}  // namespace q4
