// q4_gemv_f16.hip -- decode-time product with fp16 weights on gfx950:
// y[m, n] = sum_k x[m, k] * w[n, k] for 1 <= m <= 8 (m = 1 has a streaming
// kernel of its own, below the MFMA kernel).
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
// group (the MFMA B layout) and reads activation row r's matching eight
// elements (the A layout; rows r >= m are zero).  One MFMA per group
// accumulates D[token][row] over the whole K; the block's results are stored
// when its last step is done.  No dequantization and no per-group scaling:
// the kernel is a pure stream of 2 bytes per weight.  gemv_f16_lds_kernel
// below (activations staged in LDS, weights read in whole row segments) runs
// wherever its LDS fits; this form, which reads the activations from global
// memory at every step, serves larger k.
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

// The same product with the activations staged in LDS once per workgroup and
// the weights read in whole 256-byte row segments.  In the MFMA B layout a
// wave load covers 16 rows x 64 bytes, which streams at ~5.3 TB/s; here lane
// (lr, lj) = (lane / 16, lane % 16) loads the 16-byte chunk lj of row 4 i + lr
// (i < 4), so each wave load covers 4 rows x 256 contiguous bytes, and every
// step's 16 x 256-byte tile makes a round trip through a wave-private LDS
// tile: chunk j of row n is stored at 256 n + 16 ((j + n) mod 16), a rotation
// that keeps both the row-wise writes and the column-wise B-operand reads
// (lane (r, kq) reads chunk 4 q + kq of row r for the step's MFMA q) free of
// bank conflicts.  Two tiles per wave alternate between steps.  The k order
// inside every MFMA is the one gemv_f16_kernel uses, so the results are the
// same bits.  LDS: 9 rows of Kp halves (tokens 0..7, zero past m, and a zero
// row that A rows 8..15 read; Kp = k padded with zeros to whole steps) plus
// 8 KB per wave.  Measured on the 248,320-row heads, m = 8: k = 2560
// 326.8 -> 204 us (78% of HBM), k = 1024 117.5 -> 88 us.
constexpr int kTileBytes = 4096;                // 16 rows x 256 bytes

struct F16Tile {
    u32x4_t v[4];                               // row 4 i + lane / 16, chunk lane % 16
};

template <int PF>
__global__ __launch_bounds__(kF16Threads, 2) void gemv_f16_lds_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
    int M, int64_t N, int K, int G, int Kp, int64_t base, int64_t extra) {
    extern __shared__ __align__(16) unsigned char smem[];
    _Float16* xs = reinterpret_cast<_Float16*>(smem);
    const int cpr = Kp / 8;                                   // 16-byte chunks per LDS row
    for (int u = threadIdx.x; u < 9 * cpr; u += kF16Threads) {
        const int row = u / cpr, c = u % cpr;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (row < M && 8 * c < K)
            v = *reinterpret_cast<const u32x4_t*>(x + (int64_t)row * K + 8 * c);
        *reinterpret_cast<u32x4_t*>(xs + (int64_t)row * Kp + 8 * c) = v;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    unsigned char* tiles = smem + (size_t)9 * Kp * 2 + (size_t)wave * 2 * kTileBytes;
    const int r = lane & 15, kq = lane >> 4;                  // MFMA operand layout
    const int lr = lane >> 4, lj = lane & 15;                 // load layout
    const int64_t wv = (int64_t)blockIdx.x * kF16Waves + wave;
    const int64_t rb0 = wv * base + (wv < extra ? wv : extra);
    const int64_t cnt = base + (wv < extra ? 1 : 0);
    if (cnt <= 0) return;
    const int T = Kp / (32 * kStepGroups);                    // steps per row block
    const int64_t F = cnt * T;
    const _Float16* xa = xs + (int64_t)(r < M ? r : 8) * Kp + 8 * kq;
    // load cursor; steps past the wave's range re-read row n - 1, groups past
    // G re-read group G - 1 (their activations are zero)
    const int64_t rb_end = rb0 + cnt;
    int64_t lrb = rb0;
    int lt = 0;
    auto load_next = [&]() -> F16Tile {
        F16Tile s;
        const int g = lt * kStepGroups + (lj >> 2);
        const int gc = g < G ? g : G - 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = lrb * 16 + 4 * i + lr;
            const int64_t nc = (lrb < rb_end && n < N) ? n : N - 1;
            s.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                w + nc * (int64_t)K + 32 * gc + 8 * (lj & 3)));
        }
        const int nt = lt + 1;
        const bool wrap = nt == T;
        lt = wrap ? 0 : nt;
        lrb += wrap ? 1 : 0;
        return s;
    };
    F16Tile ring[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[p] = load_next();
    float4_t d = {0.f, 0.f, 0.f, 0.f};
    int64_t crb = rb0;
    int ct = 0;
    int tsel = 0;
    auto compute = [&](const F16Tile& s) {
        unsigned char* tile = tiles + tsel * kTileBytes;
        tsel ^= 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 4 * i + lr;
            *reinterpret_cast<u32x4_t*>(tile + 256 * n + 16 * ((lj + n) & 15)) = s.v[i];
        }
#pragma unroll
        for (int q = 0; q < kStepGroups; ++q) {
            const int c = 4 * q + kq;                         // chunk of row r
            const half8_t b =
                *reinterpret_cast<const half8_t*>(tile + 256 * r + 16 * ((c + r) & 15));
            const half8_t a =
                *reinterpret_cast<const half8_t*>(xa + 32 * (ct * kStepGroups + q));
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, d, 0, 0, 0);
        }
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

constexpr int kF16LdsMax = 160 * 1024;

size_t f16_lds_bytes(int Kp) { return (size_t)9 * Kp * 2 + (size_t)kF16Waves * 2 * kTileBytes; }

// Four steps in flight and two workgroups per CU where their LDS allows (a
// sweep of 3..8 steps x 1..3 waves per SIMD on the 248,320-row heads).
hipError_t launch_f16_lds(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                          int64_t n, int64_t k, int Kp, int cu, hipStream_t stream) {
    constexpr int PF = 4;
    const size_t lds = f16_lds_bytes(Kp);
    static std::atomic<uint64_t> lds_done{0};           // devices already set up
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(&gemv_f16_lds_kernel<PF>),
                                     (int)lds, lds_done);
    if (e != hipSuccess) return e;
    const int wps = 2 * lds <= (size_t)kF16LdsMax ? 2 : 1;
    const int64_t RB = (n + 15) / 16;
    const int64_t max_waves = (int64_t)cu * kF16Waves * wps;
    const int64_t per = (RB + max_waves - 1) / max_waves;
    const int64_t waves = (RB + per - 1) / per;
    const int blocks = (int)((waves + kF16Waves - 1) / kF16Waves);
    const int64_t W = (int64_t)blocks * kF16Waves;
    hipLaunchKernelGGL((gemv_f16_lds_kernel<PF>), dim3(blocks), dim3(kF16Threads), lds, stream,
                       x, w, y, (int)m, n, (int)k, (int)(k / 32), Kp, RB / W, RB % W);
    return hipGetLastError();
}

// m = 1: a streaming kernel without the matrix core.  LPR lanes share a row
// (RPS = 64 / LPR rows per wave step) and lane `sub` owns the 16-byte chunks
// at byte offsets 16 sub + 16 LPR i (i < CPL) of every row, so one wave load
// covers RPS rows x 16 LPR contiguous bytes and the lane's CPL activation
// chunks stay in registers for the whole kernel.  Per chunk: four
// v_dot2_f32_f16 (exact fp16 products, fp32 sums); the LPR partial sums of a
// row are added with DPP rotations.  Each wave walks its own contiguous range
// of rows with PF steps of loads in flight, refills past the range re-reading
// its last step.  (The MFMA kernel reads 16 rows x 64 bytes per wave load,
// which streams at ~5.3 TB/s; this layout streams at 6.6-6.9 TB/s.)
constexpr int kF16m1Prefetch = 2;

template <int LPR>
__device__ __forceinline__ float f16_lanes_sum(float v) {
    v = row16_sum(v);
    if (LPR >= 32) v += __shfl_xor(v, 16, 64);
    if (LPR == 64) v += __shfl_xor(v, 32, 64);
    return v;
}

template <int LPR, int CPL, int PF>
__global__ __launch_bounds__(kF16Threads) void gemv_f16_m1_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
    int64_t N, int K, int64_t base, int64_t extra) {
    constexpr int RPS = 64 / LPR;
    const int lane = threadIdx.x & 63, sub = lane % LPR, r = lane / LPR;
    const int64_t wv = (int64_t)blockIdx.x * kF16Waves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t q0 = wv * base + (wv < extra ? wv : extra);
    const int64_t cnt = base + (wv < extra ? 1 : 0);
    if (cnt <= 0) return;
    const int64_t row0 = RPS * q0 + r;
    u32x4_t rp[PF][CPL];
    auto load = [&](int slot, int64_t f) {
        int64_t row = row0 + RPS * (f < cnt ? f : cnt - 1);
        row = row < N ? row : N - 1;                 // the last step may be partial
        const uint16_t* p = w + row * (int64_t)K + 8 * sub;
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            rp[slot][i] =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + 8 * LPR * i));
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, p);
    u32x4_t xr[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        xr[i] = *reinterpret_cast<const u32x4_t*>(x + 8 * sub + 8 * LPR * i);
    auto compute = [&](int p) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            a0 = __builtin_amdgcn_fdot2(as_half2(rp[p][i][0]), as_half2(xr[i][0]), a0, false);
            a1 = __builtin_amdgcn_fdot2(as_half2(rp[p][i][1]), as_half2(xr[i][1]), a1, false);
            a0 = __builtin_amdgcn_fdot2(as_half2(rp[p][i][2]), as_half2(xr[i][2]), a0, false);
            a1 = __builtin_amdgcn_fdot2(as_half2(rp[p][i][3]), as_half2(xr[i][3]), a1, false);
        }
        return f16_lanes_sum<LPR>(a0 + a1);
    };
    auto emit = [&](float acc, int64_t f) {
        const int64_t row = row0 + RPS * f;
        if (sub == 0 && row < N) y[row] = acc;
    };
    int64_t f0 = 0;
    for (; f0 + PF < cnt; f0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const float acc = compute(p);
            load(p, f0 + p + PF);
            emit(acc, f0 + p);
        }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (f0 + p < cnt) emit(compute(p), f0 + p);
}

template <int LPR, int CPL>
hipError_t launch_f16_m1_t(const uint16_t* x, const uint16_t* w, float* y, int64_t n, int64_t k,
                           int cu, hipStream_t stream) {
    constexpr int RPS = 64 / LPR;
    const int64_t rq = (n + RPS - 1) / RPS;                  // row steps
    const int64_t max_waves = (int64_t)cu * kF16Waves;       // one wave per SIMD
    const int64_t per = (rq + max_waves - 1) / max_waves;
    const int64_t waves = (rq + per - 1) / per;
    const int blocks = (int)((waves + kF16Waves - 1) / kF16Waves);
    const int64_t W = (int64_t)blocks * kF16Waves;
    hipLaunchKernelGGL((gemv_f16_m1_kernel<LPR, CPL, kF16m1Prefetch>), dim3(blocks),
                       dim3(kF16Threads), 0, stream, x, w, y, n, (int)k, rq / W, rq % W);
    return hipGetLastError();
}

// The m = 1 configuration for k (k = 16 LPR CPL), or false when k has none.
hipError_t launch_f16_m1(const uint16_t* x, const uint16_t* w, float* y, int64_t n, int64_t k,
                         int cu, hipStream_t stream, bool& done) {
    done = true;
    if (k % 128 == 0 && k / 128 <= 8) {
        switch (k / 128) {
            case 1: return launch_f16_m1_t<16, 1>(x, w, y, n, k, cu, stream);
            case 2: return launch_f16_m1_t<16, 2>(x, w, y, n, k, cu, stream);
            case 3: return launch_f16_m1_t<16, 3>(x, w, y, n, k, cu, stream);
            case 4: return launch_f16_m1_t<16, 4>(x, w, y, n, k, cu, stream);
            case 5: return launch_f16_m1_t<16, 5>(x, w, y, n, k, cu, stream);
            case 6: return launch_f16_m1_t<16, 6>(x, w, y, n, k, cu, stream);
            case 7: return launch_f16_m1_t<16, 7>(x, w, y, n, k, cu, stream);
            default: return launch_f16_m1_t<16, 8>(x, w, y, n, k, cu, stream);
        }
    }
    if (k % 256 == 0 && k / 256 <= 10) {
        switch (k / 256) {
            case 5: return launch_f16_m1_t<32, 5>(x, w, y, n, k, cu, stream);
            case 6: return launch_f16_m1_t<32, 6>(x, w, y, n, k, cu, stream);
            case 7: return launch_f16_m1_t<32, 7>(x, w, y, n, k, cu, stream);
            case 8: return launch_f16_m1_t<32, 8>(x, w, y, n, k, cu, stream);
            case 9: return launch_f16_m1_t<32, 9>(x, w, y, n, k, cu, stream);
            default: return launch_f16_m1_t<32, 10>(x, w, y, n, k, cu, stream);
        }
    }
    if (k % 512 == 0 && k / 512 >= 6 && k / 512 <= 10) {
        switch (k / 512) {
            case 6: return launch_f16_m1_t<64, 6>(x, w, y, n, k, cu, stream);
            case 7: return launch_f16_m1_t<64, 7>(x, w, y, n, k, cu, stream);
            case 8: return launch_f16_m1_t<64, 8>(x, w, y, n, k, cu, stream);
            case 9: return launch_f16_m1_t<64, 9>(x, w, y, n, k, cu, stream);
            default: return launch_f16_m1_t<64, 10>(x, w, y, n, k, cu, stream);
        }
    }
    done = false;
    return hipSuccess;
}

}  // namespace

// m = 1: the streaming kernel where k fits it; otherwise (and for m = 2..8)
// the MFMA kernel, with each wave owning a contiguous, balanced range of row
// blocks: the LDS form while its LDS fits in 160 KB (k <= 7168), else the
// form that reads the activations from global memory.
hipError_t launch_gemv_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                           int64_t n, int64_t k, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int cu = device_info(dev).cu_count;
    if (m == 1) {
        bool done = false;
        e = launch_f16_m1(x, w, y, n, k, cu, stream, done);
        if (done) return e;
    }
    const int64_t steps = (k / 32 + kStepGroups - 1) / kStepGroups;
    const int64_t Kp = steps * 32 * kStepGroups;
    if (f16_lds_bytes((int)Kp) <= (size_t)kF16LdsMax)
        return launch_f16_lds(x, w, y, m, n, k, (int)Kp, cu, stream);
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
