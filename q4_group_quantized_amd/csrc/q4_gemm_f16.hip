// q4_gemm_f16.hip -- prefill product with fp16 weights on gfx950:
// y[m, n] = sum_t x[m, t] * w[n, t] for any m (m <= 8 goes to the decode
// kernel of q4_gemv_f16.hip).
//
// Method: the batched prefill of the QORA engines over their second weight
// format, fp16 beside Q4 (QORA-4B article, quantization section, format
// table; GPU prefill section), i.e. the F16 GEMV of the QORA-LLM-0.8B model
// card ("AVX-512 SIMD Acceleration", F16 GEMV row) for a whole token batch.
//
// Arithmetic.  fp16 weights are the B operand of v_mfma_f32_16x16x32_f16 as
// they stand, activations the A operand; every product of two fp16 values is
// exact and each 16x16 output block accumulates in fp32 over all of K in the
// matrix core itself -- no dequantization and no per-group scale.
//
// Work split and data movement follow the Q4 GEMM: a workgroup owns a
// BM x (32*WN) tile of y; its waves are WN column slices of 32 x WK slices of
// K; every operand goes straight from global memory into LDS with
// direct-to-LDS loads through an S-stage ring, 16 rows x 64 bytes (one
// 32-wide K step of 16 rows) per wave instruction, for the activations and
// the weight rows alike; each lane reads an operand with one ds_read_b128.
// The WK partial tiles are added in LDS in a fixed order (deterministic).
// Rows past M or N and K steps past K/32 are clamped to real addresses: their
// results are never stored.  K steps past the end of a wave's K slice read
// both operands from a block of zeros in LDS, so they add exactly 0 and the
// loop has no per-step branch.
#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kF16Block = 1024;            // 16 rows x 32 halves

__device__ __forceinline__ constexpr int f16_vmcnt_imm(int n) {
    // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 (gfx9)
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

template <int BM, int WN, int WK, int KG, int S>
struct GemmF16 {
    static constexpr int MB = BM / 16;                 // 16-row blocks of x per wave
    static constexpr int BN = 32 * WN;
    static constexpr int NB = BN / 16;                 // 16-row blocks of w per tile
    static constexpr int kWOff = KG * MB * kF16Block;  // weights after activations
    static constexpr int kStageBytes = kWOff + KG * NB * kF16Block;
    static constexpr int kABlocksPerWave = KG * MB / WN;
    static constexpr int kWBlocksPerWave = KG * NB / WN;
    static constexpr int kLoadsPerStage = kABlocksPerWave + kWBlocksPerWave;
    static constexpr int kLdsBytes = WK * S * kStageBytes;
    // zeros that the operand reads of out-of-range K steps are pointed at
    static constexpr int kZeroBytes = (MB > NB ? MB : NB) * kF16Block;
    static constexpr int kLdsTotal = kLdsBytes + kZeroBytes;
    static constexpr int kRedBytes = (WK - 1) * WN * MB * 8 * 64 * 4;
    static constexpr int kThreads = 64 * WN * WK;
    static_assert(WN * WK == 4 || WN * WK == 8, "one or two waves per SIMD");
    static_assert((KG * MB) % WN == 0, "activation blocks split evenly");
    static_assert(S >= 2, "at least double buffering");
    static_assert(kRedBytes <= kLdsBytes, "reduction fits in the staging space");
    static_assert(kLdsTotal <= 160 * 1024, "LDS of one CU");
};

// Workgroups per launch at most (the dispatch counts work-items in 32 bits);
// larger tile counts take several launches, each from its own first tile.
constexpr int64_t kGemmF16MaxGrid = 1 << 20;

// At least two waves per SIMD: caps a wave at 256 registers, which keeps the
// MFMA accumulators in VGPRs.
template <int BM, int WN, int WK, int KG, int S>
__global__ __launch_bounds__(64 * WN * WK, 2) void gemm_f16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
    int M, int64_t N, int K, int G, int64_t tiles_n, int64_t tile_base) {
    using C = GemmF16<BM, WN, WK, KG, S>;
    constexpr int MB = C::MB;
    extern __shared__ __align__(16) unsigned char smem[];

    const int64_t tile = tile_base + blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar branches
    const int wn = wave % WN;
    const int kp = wave / WN;
    const int64_t nt0 = (tile % tiles_n) * C::BN;     // tile's first column
    const int64_t m0 = (tile / tiles_n) * BM;

    const int Gp = (G + WK - 1) / WK;                 // K steps per K slice
    const int gbeg = kp * Gp;
    const int gend = min(G, gbeg + Gp);
    const int nstages = (Gp + KG - 1) / KG;           // same for every wave

    unsigned char* kbase = smem + (size_t)kp * S * C::kStageBytes;
    // zero operands for K steps past the slice's end (both operands: a zero
    // weight times an infinite activation, or the reverse, would be NaN)
    const unsigned char* zero = smem + C::kLdsBytes;
    for (int i = threadIdx.x; i < C::kZeroBytes / 16; i += C::kThreads)
        reinterpret_cast<u32x4_t*>(smem + C::kLdsBytes)[i] = u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0): zeros stored before the first barrier
    // Workgroups start their walk over K at a stage set by their column tile:
    // tiles of different columns spread their requests for the same activation
    // rows over K, while the row tiles of one column walk its weights in step
    // and share them in L2 (fp16 weights far exceed it).  The order of the
    // fp32 sums depends only on the tile index, identically on every run.
    const int rot = (int)((tile % tiles_n) % nstages);
    auto stage_step = [&](int st) {               // first K step (in the slice) of stage st
        const int r = st + rot;
        return (r < nstages ? r : r - nstages) * KG;
    };

    // load-side lane mapping: 16 rows x 4 16-byte parts per instruction
    const int l_row = lane >> 2, l_part = lane & 3;
    // operand-side lane mapping
    const int col = lane & 15, kq = lane >> 4;

    auto issue = [&](int st, int buf) {
        unsigned char* sb = kbase + buf * C::kStageBytes;
        const int gs = gbeg + stage_step(st);
#pragma unroll
        for (int i = 0; i < C::kABlocksPerWave; ++i) {
            const int b = wn * C::kABlocksPerWave + i;
            const int gl = b / MB, mb = b % MB;
            const int g = min(gs + gl, G - 1);
            const int64_t r = min<int64_t>(m0 + 16 * mb + l_row, M - 1);
            __builtin_amdgcn_global_load_lds(x + r * K + 32 * g + 8 * l_part,
                                             (lds_void_t*)(sb + (gl * MB + mb) * kF16Block),
                                             16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::kWBlocksPerWave; ++i) {
            const int b = wn * C::kWBlocksPerWave + i;
            const int gl = b / C::NB, nbk = b % C::NB;
            const int g = min(gs + gl, G - 1);
            const int64_t r = min<int64_t>(nt0 + 16 * nbk + l_row, N - 1);
            __builtin_amdgcn_global_load_lds(
                w + r * K + 32 * g + 8 * l_part,
                (lds_void_t*)(sb + C::kWOff + (gl * C::NB + nbk) * kF16Block), 16, 0, 0);
        }
    };

    float4_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < S - 1; ++u) issue(u, u);

    // operands of one K step, read from LDS one step ahead of their MFMAs
    struct Ops {
        half8_t a[MB];
        half8_t b[2];
    };
    auto read_ops = [&](Ops& o, const unsigned char* sb, int gl, bool valid) {
        const unsigned char* ab = valid ? sb + gl * MB * kF16Block : zero;
        const unsigned char* bb = valid ? sb + C::kWOff + gl * C::NB * kF16Block : zero;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            o.a[mb] = *reinterpret_cast<const half8_t*>(ab + mb * kF16Block + 64 * col + 16 * kq);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            o.b[nb] = *reinterpret_cast<const half8_t*>(bb + (2 * wn + nb) * kF16Block +
                                                        64 * col + 16 * kq);
    };
    auto compute = [&](const Ops& o) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                acc[mb][nb] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(o.a[mb], o.b[nb], acc[mb][nb], 0, 0, 0);
    };

    for (int st0 = 0; st0 < nstages; st0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int st = st0 + u;
            if (st < nstages) {
                // stage st has landed once at most the S-2 later stages remain
                // in flight (every wave issues the same number of loads)
                __builtin_amdgcn_s_waitcnt(f16_vmcnt_imm(C::kLoadsPerStage * (S - 2)));
                barrier_keep_loads();
                // refill the buffer computed last iteration (every wave is past it)
                issue(st + S - 1, (u + S - 1) % S);
                const unsigned char* sb = kbase + u * C::kStageBytes;
                const int g0 = gbeg + stage_step(st);
                Ops ops[2];
                read_ops(ops[0], sb, 0, g0 < gend);
#pragma unroll
                for (int gl = 0; gl < KG; ++gl) {
                    if (gl + 1 < KG) read_ops(ops[(gl + 1) & 1], sb, gl + 1, g0 + gl + 1 < gend);
                    compute(ops[gl & 1]);
                }
            }
        }
    }

    // add the K slices: slices 1..WK-1 park their partial tiles in LDS, slice
    // 0 adds them in slice order and stores
    __builtin_amdgcn_s_waitcnt(f16_vmcnt_imm(0));
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    if (kp > 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[((((kp - 1) * WN + wn) * MB + mb) * 8 + nb * 4 + v) * 64 + lane] =
                        acc[mb][nb][v];
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int64_t n = nt0 + 32 * wn + 16 * nb + col;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float t = acc[mb][nb][v];
#pragma unroll
                    for (int q = 1; q < WK; ++q)
                        t += red[((((q - 1) * WN + wn) * MB + mb) * 8 + nb * 4 + v) * 64 + lane];
                    const int64_t m = m0 + 16 * mb + 4 * kq + v;
                    if (m < M && n < N) y[m * N + n] = t;
                }
            }
    }
}

template <int BM, int WN, int WK, int KG, int S>
hipError_t launch_gemm_f16_t(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                             int64_t n, int64_t k, hipStream_t stream) {
    using C = GemmF16<BM, WN, WK, KG, S>;
    const int64_t tiles_n = (n + C::BN - 1) / C::BN;
    const int64_t tiles = tiles_n * ((m + BM - 1) / BM);
    static std::atomic<uint64_t> lds_done{0};           // devices already set up
    hipError_t e = allow_dynamic_lds(
        reinterpret_cast<const void*>(&gemm_f16_kernel<BM, WN, WK, KG, S>), C::kLdsTotal, lds_done);
    if (e != hipSuccess) return e;
    for (int64_t base = 0; base < tiles; base += kGemmF16MaxGrid) {
        const int64_t grid = tiles - base < kGemmF16MaxGrid ? tiles - base : kGemmF16MaxGrid;
        hipLaunchKernelGGL((gemm_f16_kernel<BM, WN, WK, KG, S>), dim3((unsigned)grid),
                           dim3(C::kThreads), C::kLdsTotal, stream, x, w, y, (int)m, n, (int)k,
                           (int)(k / 32), tiles_n, base);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemm_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                           int64_t n, int64_t k, hipStream_t stream) {
    if (m <= 8) return launch_gemv_f16(x, w, y, m, n, k, stream);
    if (m <= 16) return launch_gemm_f16_t<16, 1, 4, 2, 4>(x, w, y, m, n, k, stream);
    if (m <= 32) return launch_gemm_f16_t<32, 1, 4, 2, 4>(x, w, y, m, n, k, stream);
    // above, the tile shape with the least estimated time (choose_tile); the
    // 128- and 64-column-wide shapes without a K split pay with 3.6x the weight
    // bytes of Q4 (fewer weight re-reads per output).  Round times measured
    // at k = 2560, n = 4096, one tile per CU.
    static constexpr TileChoice kTilesF16[] = {
        {128, 128, 38.5f},     // gemm_f16_kernel<128, 4, 1, 1, 8>
        {64, 128, 23.6f},      // gemm_f16_kernel<64, 4, 1, 2, 4>
        {64, 64, 19.6f},       // gemm_f16_kernel<64, 2, 4, 2, 2>
        {32, 64, 16.2f},       // gemm_f16_kernel<32, 2, 4, 2, 2>
    };
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    switch (choose_tile(kTilesF16, 4, m, 1, &n, device_info(dev).cu_count)) {
        case 0: return launch_gemm_f16_t<128, 4, 1, 1, 8>(x, w, y, m, n, k, stream);
        case 1: return launch_gemm_f16_t<64, 4, 1, 2, 4>(x, w, y, m, n, k, stream);
        case 2: return launch_gemm_f16_t<64, 2, 4, 2, 2>(x, w, y, m, n, k, stream);
        default: return launch_gemm_f16_t<32, 2, 4, 2, 2>(x, w, y, m, n, k, stream);
    }
}

}  // namespace q4
