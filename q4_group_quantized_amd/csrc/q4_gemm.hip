// q4_gemm.hip -- prefill Q4 product y = x * dequant(W)^T for many tokens on gfx950.
//
// Method: the batched prefill of the QORA pages, where every projection of a
// token batch is one matrix product over 4-bit weights (QORA-4B article, GPU
// prefill section; QORA-LLM-0.8B model card, "Performance"), with the Q4
// format of their quantization sections (symmetric, group size 32, 16-entry
// table dequantization).
//
// Tiling.  A workgroup owns a BM x BN tile of y and walks K two groups (64
// elements) per stage.  Each stage stages through LDS, double-buffered:
//   - the BM x 64 activation tile, permuted inside every 8-element chunk to
//     the order in which unpack8 emits codes;
//   - the BN x 32 packed-code tile (raw nibbles, 0.5 byte per weight);
//   - the BN x 2 fp16 scales.
// Global loads of stage s+1 are issued before the MFMAs of stage s.
//
// Per group, each wave turns one packed dword per lane into eight exact fp16
// levels -8..7 (the table lookup, see q4_device.hpp), runs one
// v_mfma_f32_16x16x32_f16 per 16x16 block with a zero accumulator -- K = 32 is
// exactly one group -- and folds the result into its fp32 accumulators with
// the group's scale: acc += s[n, j] * P.  In the 16x16 D layout a lane's four
// values share one column, hence one scale.
#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {
namespace {

constexpr int kKG = 2;                               // groups per stage
constexpr int kXRow = kKG * 32 + 8;                  // halves per LDS row (padded)
constexpr int kWRow = kKG * 16 + 4;                  // bytes per LDS row (padded)

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
    static constexpr int kThreads = 64 * WM * WN;
    static constexpr int TM = BM / WM;               // wave tile
    static constexpr int TN = BN / WN;
    static constexpr int MB = TM / 16;               // MFMA blocks per wave
    static constexpr int NB = TN / 16;
    static constexpr int kXUnits = BM * kKG * 4;     // 16-byte units per stage
    static constexpr int kWUnits = BN * kKG;
    static constexpr int kSUnits = BN * kKG;
    static constexpr int kXPer = (kXUnits + kThreads - 1) / kThreads;
    static constexpr int kWPer = (kWUnits + kThreads - 1) / kThreads;
    static constexpr int kSPer = (kSUnits + kThreads - 1) / kThreads;
    static_assert(MB >= 1 && NB >= 1, "wave tile below one MFMA block");
};

template <class C>
struct StageRegs {
    u32x4_t xv[C::kXPer];
    u32x4_t wv[C::kWPer];
    uint32_t sv[C::kSPer];
};

template <int BM, int BN, class C>
__device__ __forceinline__ void load_stage(StageRegs<C>& r, const uint16_t* __restrict__ x,
                                           const uint8_t* __restrict__ packed,
                                           const uint16_t* __restrict__ scales,
                                           int64_t m0, int64_t n0, int M, int64_t N,
                                           int K, int G, int j0) {
#pragma unroll
    for (int i = 0; i < C::kXPer; ++i) {
        const int u = threadIdx.x + i * C::kThreads;
        r.xv[i] = u32x4_t{0u, 0u, 0u, 0u};
        if (u < C::kXUnits) {
            const int row = u / (kKG * 4);
            const int rest = u % (kKG * 4);
            const int j = j0 + rest / 4;
            const int64_t m = m0 + row;
            if (m < M && j < G)
                r.xv[i] = *reinterpret_cast<const u32x4_t*>(x + m * K + 32 * j + 8 * (rest & 3));
        }
    }
#pragma unroll
    for (int i = 0; i < C::kWPer; ++i) {
        const int u = threadIdx.x + i * C::kThreads;
        r.wv[i] = u32x4_t{0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
        if (u < C::kWUnits) {
            const int row = u / kKG;
            const int j = j0 + u % kKG;
            const int64_t n = n0 + row;
            if (n < N && j < G)
                r.wv[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(packed + n * (K / 2) + 16 * j));
        }
    }
#pragma unroll
    for (int i = 0; i < C::kSPer; ++i) {
        const int u = threadIdx.x + i * C::kThreads;
        r.sv[i] = 0u;
        if (u < C::kSUnits) {
            const int row = u / kKG;
            const int j = j0 + u % kKG;
            const int64_t n = n0 + row;
            if (n < N && j < G) r.sv[i] = scales[n * G + j];
        }
    }
}

template <int BM, int BN, class C>
__device__ __forceinline__ void store_stage(const StageRegs<C>& r, _Float16* xs, uint8_t* ws,
                                            uint16_t* ss) {
#pragma unroll
    for (int i = 0; i < C::kXPer; ++i) {
        const int u = threadIdx.x + i * C::kThreads;
        if (u < C::kXUnits) {
            const int row = u / (kKG * 4);
            const int rest = u % (kKG * 4);
            *reinterpret_cast<u32x4_t*>(xs + row * kXRow + 8 * rest) = permute_x8(r.xv[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < C::kWPer; ++i) {
        const int u = threadIdx.x + i * C::kThreads;
        if (u < C::kWUnits) {
            const int row = u / kKG;
            uint32_t* dst = reinterpret_cast<uint32_t*>(ws + row * kWRow + 16 * (u % kKG));
#pragma unroll
            for (int q = 0; q < 4; ++q) dst[q] = r.wv[i][q];
        }
    }
#pragma unroll
    for (int i = 0; i < C::kSPer; ++i) {
        const int u = threadIdx.x + i * C::kThreads;
        if (u < C::kSUnits) ss[(u % kKG) * BN + u / kKG] = (uint16_t)r.sv[i];
    }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int M, int64_t N,
    int K, int G) {
    using C = GemmCfg<BM, BN, WM, WN>;
    __shared__ __align__(16) _Float16 xs[2][BM * kXRow];
    __shared__ __align__(16) uint8_t ws[2][BN * kWRow];
    __shared__ __align__(16) uint16_t ss[2][kKG * BN];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t n0 = ((int64_t)blockIdx.x % tiles_n) * BN;
    const int64_t m0 = ((int64_t)blockIdx.x / tiles_n) * BM;
    const int col = lane & 15, kq = lane >> 4;

    float4_t acc[C::MB][C::NB];
#pragma unroll
    for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    const int stages = (G + kKG - 1) / kKG;
    StageRegs<C> regs;
    load_stage<BM, BN, C>(regs, x, packed, scales, m0, n0, M, N, K, G, 0);
    store_stage<BM, BN, C>(regs, xs[0], ws[0], ss[0]);
    __syncthreads();

    for (int s = 0; s < stages; ++s) {
        const int buf = s & 1;
        if (s + 1 < stages)
            load_stage<BM, BN, C>(regs, x, packed, scales, m0, n0, M, N, K, G, (s + 1) * kKG);
#pragma unroll
        for (int g = 0; g < kKG; ++g) {
            half8_t a[C::MB];
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
                a[mb] = *reinterpret_cast<const half8_t*>(
                    &xs[buf][(wm * C::TM + mb * 16 + col) * kXRow + g * 32 + 8 * kq]);
            half8_t b[C::NB];
            float sc[C::NB];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                const int r = wn * C::TN + nb * 16 + col;
                b[nb] = unpack8(*reinterpret_cast<const uint32_t*>(
                    &ws[buf][r * kWRow + g * 16 + 4 * kq]));
                sc[nb] = half_bits_to_float(ss[buf][g * BN + r]);
            }
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    const float4_t zero = {0.f, 0.f, 0.f, 0.f};
                    float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], b[nb], zero, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[mb][nb][v] = fmaf(sc[nb], p[v], acc[mb][nb][v]);
                }
        }
        if (s + 1 < stages)
            store_stage<BM, BN, C>(regs, xs[buf ^ 1], ws[buf ^ 1], ss[buf ^ 1]);
        __syncthreads();
    }

#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            const int64_t n = n0 + wn * C::TN + nb * 16 + col;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t m = m0 + wm * C::TM + mb * 16 + 4 * kq + v;
                if (m < M && n < N) y[m * N + n] = acc[mb][nb][v];
            }
        }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_gemm_t(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                         float* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
    const int64_t tiles = ((n + BN - 1) / BN) * ((m + BM - 1) / BM);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN>), dim3((unsigned)tiles),
                       dim3(64 * WM * WN), 0, stream, x, packed, scales, y, (int)m, n,
                       (int)k, (int)(k / 32));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                       float* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
    if (m <= 8) return launch_gemv(x, packed, scales, y, m, n, k, stream);
    if (m <= 16) return launch_gemm_t<16, 64, 1, 4>(x, packed, scales, y, m, n, k, stream);
    if (m < 128) return launch_gemm_t<64, 64, 2, 2>(x, packed, scales, y, m, n, k, stream);
    return launch_gemm_t<128, 64, 2, 2>(x, packed, scales, y, m, n, k, stream);
}

}  // namespace q4
