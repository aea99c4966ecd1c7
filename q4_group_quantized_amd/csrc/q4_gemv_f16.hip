// q4_gemv_f16.hip -- decode-time product with fp16 weights on gfx950:
// y[m, n] = sum_k x[m, k] * w[n, k] for 1 <= m <= 8.
//
// Method: the F16 GEMV of the QORA engines, their second weight format beside
// Q4 (QORA-4B article, quantization section, format table; QORA-LLM-0.8B
// model card, "AVX-512 SIMD Acceleration", F16 GEMV row: each fp16 weight is
// widened and multiply-accumulated).  On CDNA4 the widening is free: fp16
// weights are the B operand of v_mfma_f32_16x16x32_f16 as they stand, and
// every product of two fp16 values is exact in the fp32 accumulator.
//
// Work split.  A wave owns a contiguous range of 16-row blocks and walks each
// block's K in steps of four 32-element groups (16 rows x 256 bytes: whole
// cache lines), with PF steps of loads in flight.  Lane (r, kq) = (lane % 16,
// lane / 16) loads weight row r's eight elements at K offset 8 kq of every
// group (the MFMA B layout) and activation row r's matching eight elements
// (the A layout; rows r >= m read nothing and stay zero).  One MFMA per group
// accumulates D[token][row] over the whole K; the block's results are stored
// when its last step is done.  No dequantization and no per-group scaling:
// the kernel is a pure stream of 2 bytes per weight.
#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {
namespace {

constexpr int kF16Waves = 4;
constexpr int kF16Threads = 64 * kF16Waves;
constexpr int kStepGroups = 4;          // 32-element groups per step
constexpr int kF16Prefetch = 4;         // steps in flight per wave

struct F16Step {
    half8_t w[kStepGroups];             // B operands
    half8_t x[kStepGroups];             // A operands
};

// Wave w of the grid owns row blocks [w * base + min(w, extra), +base + (w < extra)).
// Refill loads past the wave's last step re-read that step (its own rows), so
// every load is unconditional and PF steps stay in flight; the last PF steps
// are computed after the loop.
template <int PF>
__global__ __launch_bounds__(kF16Threads, 1) void gemv_f16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
    int M, int64_t N, int K, int G, int64_t base, int64_t extra) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, kq = lane >> 4;
    const int64_t wv = (int64_t)blockIdx.x * kF16Waves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t rb0 = wv * base + (wv < extra ? wv : extra);
    const int64_t cnt = base + (wv < extra ? 1 : 0);
    if (cnt <= 0) return;
    const int T = (G + kStepGroups - 1) / kStepGroups;       // steps per row block
    const int64_t F = cnt * T;
    const bool tok = r < M;                                    // this lane's A row is a token
    const uint16_t* xrow = x + (int64_t)(tok ? r : 0) * K + 8 * kq;

    // load cursor: (row block, step), held at the wave's last step once reached
    int64_t lrb = rb0, lf = 0;
    int lt = 0;
    auto load_next = [&]() -> F16Step {
        F16Step s;
        int64_t n = lrb * 16 + r;
        n = n < N ? n : N - 1;
        const uint16_t* wrow = w + n * (int64_t)K + 8 * kq;
#pragma unroll
        for (int q = 0; q < kStepGroups; ++q) {
            const int g = lt * kStepGroups + q;
            const int gc = g < G ? g : G - 1;
            s.w[q] = __builtin_nontemporal_load(reinterpret_cast<const half8_t*>(wrow + 32 * gc));
            s.x[q] = half8_t{};
            if (tok && g < G) s.x[q] = *reinterpret_cast<const half8_t*>(xrow + 32 * g);
        }
        if (lf + 1 < F) {
            ++lf;
            if (++lt == T) { lt = 0; ++lrb; }
        }
        return s;
    };

    F16Step ring[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[p] = load_next();

    float4_t d = {0.f, 0.f, 0.f, 0.f};
    int64_t crb = rb0;
    int ct = 0;
    auto compute = [&](const F16Step& s) {
#pragma unroll
        for (int q = 0; q < kStepGroups; ++q)
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(s.x[q], s.w[q], d, 0, 0, 0);
        if (++ct == T) {
            // D[4 kq + v][r]: token 4 kq + v, weight row 16 crb + r
            const int64_t n = crb * 16 + r;
            if (n < N) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int t = 4 * kq + v;
                    if (t < M) y[(int64_t)t * N + n] = d[v];
                }
            }
            d = float4_t{0.f, 0.f, 0.f, 0.f};
            ct = 0;
            ++crb;
        }
    };

    int64_t f0 = 0;
    for (; f0 + PF < F; f0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            compute(ring[p]);
            ring[p] = load_next();
        }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (f0 + p < F) compute(ring[p]);
}

}  // namespace

// One wave per SIMD, each with a contiguous, balanced range of row blocks.
hipError_t launch_gemv_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                           int64_t n, int64_t k, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int64_t RB = (n + 15) / 16;
    const int64_t max_waves = (int64_t)device_info(dev).cu_count * kF16Waves;
    const int64_t per = (RB + max_waves - 1) / max_waves;
    const int64_t waves = (RB + per - 1) / per;
    const int blocks = (int)((waves + kF16Waves - 1) / kF16Waves);
    const int64_t W = (int64_t)blocks * kF16Waves;
    hipLaunchKernelGGL((gemv_f16_kernel<kF16Prefetch>), dim3(blocks), dim3(kF16Threads), 0,
                       stream, x, w, y, (int)m, n, (int)k, (int)(k / 32), RB / W, RB % W);
    return hipGetLastError();
}

}  // namespace q4
