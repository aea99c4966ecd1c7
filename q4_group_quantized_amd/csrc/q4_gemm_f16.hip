// q4_gemm_f16.hip -- prefill product with fp16 weights on gfx950:
// y[m, n] = sum_t x[m, t] * w[n, t] for any m (m <= 8 goes to the decode
// kernel of q4_gemv_f16.hip).
//
// Method: the batched prefill of the QORA engines over their second weight
// format, fp16 beside Q4 (QORA-4B article, quantization section, format
// table; GPU prefill section), i.e. the F16 GEMV of the QORA-LLM-0.8B model
// card ("AVX-512 SIMD Acceleration", F16 GEMV row) for a whole token batch.
//
// Arithmetic.  fp16 weights are the B operand of the MFMA as they stand,
// activations the A operand; every product of two fp16 values is exact and
// each output block accumulates in fp32 over all of K in the matrix core
// itself -- no dequantization and no per-group scale.
//
// Two kernels: m <= 32 runs gemm_f16_kernel (16 x 16 blocks,
// v_mfma_f32_16x16x32_f16, described next); m > 32 runs gemm32_f16_kernel
// further down (32 x 32 blocks, whole-row staging of both operands).
//
// gemm_f16_kernel.  Work split and data movement follow the Q4 GEMM: a workgroup owns a
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

// ---------------------------------------------------------------------------
// m > 32: 32 x 32 output blocks (v_mfma_f32_32x32x16_f16)
//
// Both operands are rows of fp16 with K contiguous (x[m][t], w[n][t]), so
// they are staged alike: a stage holds KG consecutive 32-wide K steps
// ("groups") of the tile's BM activation rows followed by its BN weight rows,
// each row's KG * 64 bytes contiguous in LDS.  Every wave instruction loads
// whole row slices (64 / (4 KG) rows x 64 KG bytes, i.e. 4 rows x 256 bytes
// at KG = 4) straight into LDS; the 16-byte chunk c of stage row r sits at
// position c ^ (r & 7) of its row, so that the operand reads of a wave touch
// distinct banks.  The MFMAs accumulate over all of K in place: no
// dequantization and no per-group scale, so the loop issues no VALU work.
//
// Work split.  WM x WN x WK waves: wave (wm, wn, wk) computes the 32 MB x
// 32 NB block of y at rows 32 MB wm, columns 32 NB wn, over the groups wk,
// wk + WK, ... of every stage.  The WK partial tiles are added in LDS in a
// fixed order (deterministic for a given m, n, k).
// K mapping inside a group: lane (i, g) (i = lane % 32, g = lane / 32) feeds
// MFMA h (h = 0, 1) with the 8 elements of chunk 2g + h, of activation row i
// and of weight row i alike.
// ---------------------------------------------------------------------------
typedef float f16x32_acc_t __attribute__((ext_vector_type(16)));
typedef uint32_t f16x32_u32x16_t __attribute__((ext_vector_type(16)));

template <int MB, int NB, int WM, int WN, int WK, int KG, int S>
struct F16x32 {
    static constexpr int BM = 32 * MB * WM;
    static constexpr int BN = 32 * NB * WN;
    static constexpr int W = WM * WN * WK;
    static constexpr int kThreads = 64 * W;
    static constexpr int GPW = KG / WK;                  // groups per wave and stage
    static constexpr int kRowBytes = KG * 64;            // one row's slice of a stage
    static constexpr int kABytes = BM * kRowBytes;
    static constexpr int kStage = (BM + BN) * kRowBytes;
    static constexpr int NL = kStage / 1024;             // load instructions per stage
    static constexpr int NLW = NL / W;                   // ... per wave
    static constexpr int RS = BN + 4;                    // floats per row of a partial tile
    static constexpr int kRedBytes = WK * BM * RS * 4;
    static constexpr int kLds = S * kStage > kRedBytes ? S * kStage : kRedBytes;
    static constexpr int CPR = 4 * KG;                   // 16-byte chunks per stage row
    static constexpr int RPI = 64 / CPR;                 // stage rows per load instruction
    static_assert(KG % WK == 0, "whole groups per wave");
    static_assert(KG == 2 || KG == 4 || KG == 8 || KG == 16, "power-of-two stage");
    static_assert(NL % W == 0, "equal loads per wave");
    static_assert(NLW <= 16, "load offsets fit one vector");
    static_assert(BM % RPI == 0, "a load instruction reads one operand only");
    static_assert(W == 4 || W == 8, "one or two waves per SIMD");
    static_assert(S >= 2, "at least double buffering");
    static_assert(kLds <= 160 * 1024, "LDS of one CU");
};

template <int MB, int NB, int WM, int WN, int WK, int KG, int S, bool TAIL>
__global__ __launch_bounds__(64 * WM * WN * WK, 1) void gemm32_f16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, float* __restrict__ y,
    int M, int64_t N, int K, int G, int64_t tiles_n, int64_t tile_base, int vec_store) {
    using C = F16x32<MB, NB, WM, WN, WK, KG, S>;
    extern __shared__ __align__(16) unsigned char smem[];

    const int64_t tile = tile_base + blockIdx.x;
    const int64_t n0 = (tile % tiles_n) * C::BN;
    const int64_t m0 = (tile / tiles_n) * C::BM;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM, wn = (wave / WM) % WN, wk = wave / (WM * WN);
    const int li = lane & 31, lg = lane >> 5;
    const int nstages = (G + KG - 1) / KG;

    // ---- per-lane load offsets: instruction t of this wave reads stage rows
    // RPI q .. RPI q + RPI - 1 (q = wave * NLW + t), activation rows below BM,
    // weight rows from BM on; rows past M or N are clamped to the last one ----
    f16x32_u32x16_t off = {};
    uint32_t isw = 0;                                   // bit t: instruction t reads weights
    int grp[C::NLW];                                    // group of the stage each lane loads
#pragma unroll
    for (int t = 0; t < C::NLW; ++t) {
        const int q = wave * C::NLW + t;
        const int r = q * C::RPI + lane / C::CPR;
        const int c = (lane % C::CPR) ^ (r & 7);
        int64_t row;
        if (q * C::RPI < C::BM) {
            row = min<int64_t>(m0 + r, M - 1) - m0;
        } else {
            row = min<int64_t>(n0 + (r - C::BM), N - 1) - n0;
            isw |= 1u << t;
        }
        grp[t] = c >> 2;
        off[t] = (uint32_t)(row * K * 2) + (uint32_t)(c * 16);
    }
    const unsigned char* xbase = reinterpret_cast<const unsigned char*>(x + m0 * K);
    const unsigned char* wbase = reinterpret_cast<const unsigned char*>(w + n0 * K);

    // Loads of stage st into ring buffer buf.  With TAIL (G not a multiple of
    // KG), groups past G in the last stage re-read group G - 1 (in bounds;
    // their products are never computed).
    auto issue = [&](int st, int buf) {
        unsigned char* sb = smem + buf * C::kStage;
        const int g0 = st * KG;
        const int over = g0 - (G - 1);
#pragma unroll
        for (int t = 0; t < C::NLW; ++t) {
            const uint32_t back = TAIL ? (uint32_t)max(0, over + grp[t]) * 64u : 0u;
            const unsigned char* base = ((isw >> t) & 1u) ? wbase : xbase;
            __builtin_amdgcn_global_load_lds(base + (size_t)g0 * 64 + (off[t] - back),
                                             (lds_void_t*)(sb + (wave * C::NLW + t) * 1024),
                                             16, 0, 0);
        }
    };

    // ---- per-lane operand offsets inside a stage ----
    int rA[C::GPW][2], rB[C::GPW][2];
#pragma unroll
    for (int u = 0; u < C::GPW; ++u) {
        const int gl = wk + WK * u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int pos = ((gl * 4 + 2 * lg + h) ^ (li & 7)) * 16;
            rA[u][h] = (32 * MB * wm + li) * C::kRowBytes + pos;
            rB[u][h] = C::kABytes + (32 * NB * wn + li) * C::kRowBytes + pos;
        }
    }

    f16x32_acc_t acc[MB][NB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rb][nb][v] = 0.f;

    struct Ops {
        half8_t a[MB][2];
        half8_t b[NB][2];
    };
    auto read_ops = [&](Ops& o, const unsigned char* sb, int u) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
                o.a[rb][h] = *reinterpret_cast<const half8_t*>(sb + rA[u][h] +
                                                               rb * 32 * C::kRowBytes);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                o.b[nb][h] = *reinterpret_cast<const half8_t*>(sb + rB[u][h] +
                                                               nb * 32 * C::kRowBytes);
        }
    };
    auto mfmas = [&](const Ops& o) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[rb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.a[rb][h], o.b[nb][h],
                                                                         acc[rb][nb], 0, 0, 0);
    };
    // every wave's groups of one stage, operands read one group ahead
    auto stage = [&](const unsigned char* sb) {
        Ops ops[2];
        read_ops(ops[0], sb, 0);
#pragma unroll
        for (int u = 0; u < C::GPW; ++u) {
            if (u + 1 < C::GPW) read_ops(ops[(u + 1) & 1], sb, u + 1);
            mfmas(ops[u & 1]);
        }
    };

    // Every iteration issues one stage's loads (stages past the end re-load
    // the last one into a buffer nobody reads again), so stage st has landed
    // once at most S - 2 later stages' loads remain in flight; after the
    // barrier every wave's loads of it have landed, and every wave is done
    // with the buffer that the refill overwrites.
    auto wait_stage = [&]() {
        __builtin_amdgcn_s_waitcnt(f16_vmcnt_imm(C::NLW * (S - 2)));
        barrier_keep_loads();
    };
#pragma unroll
    for (int u = 0; u < S - 1; ++u) issue(min(u, nstages - 1), u);

    const int nfull = G / KG;
    int st = 0;
    for (; st + S <= nfull; st += S) {
#pragma unroll
        for (int b = 0; b < S; ++b) {
            wait_stage();
            issue(min(st + b + S - 1, nstages - 1), (b + S - 1) % S);
            stage(smem + b * C::kStage);
        }
    }
    for (; st < nfull; ++st) {
        const int b = st % S;
        wait_stage();
        issue(min(st + S - 1, nstages - 1), (b + S - 1) % S);
        stage(smem + b * C::kStage);
    }
    if (TAIL && nfull < nstages) {          // the partial last stage: its real groups only
        const int b = nfull % S;
        wait_stage();
        const unsigned char* sb = smem + b * C::kStage;
#pragma unroll
        for (int u = 0; u < C::GPW; ++u)
            if (nfull * KG + wk + WK * u < G) {
                Ops o;
                read_ops(o, sb, u);
                mfmas(o);
            }
    }

    // ---- add the WK partial tiles (fixed order) and store ----
    __builtin_amdgcn_s_waitcnt(f16_vmcnt_imm(0));
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    {
        float* dst = red + wk * C::BM * C::RS + (32 * MB * wm) * C::RS + 32 * NB * wn + li;
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    dst[(32 * rb + 8 * (v >> 2) + 4 * lg + (v & 3)) * C::RS + 32 * nb] =
                        acc[rb][nb][v];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < C::BM * C::BN / 4; i += C::kThreads) {
        const int r = i / (C::BN / 4), c = 4 * (i % (C::BN / 4));
        const int64_t m = m0 + r, n = n0 + c;
        if (m >= M) continue;
        f32x4_t t = *reinterpret_cast<const f32x4_t*>(red + r * C::RS + c);
#pragma unroll
        for (int q = 1; q < WK; ++q)
            t += *reinterpret_cast<const f32x4_t*>(red + q * C::BM * C::RS + r * C::RS + c);
        float* out = y + m * N + n;
        if (vec_store && n + 3 < N) {
            *reinterpret_cast<f32x4_t*>(out) = t;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < N) out[e] = t[e];
        }
    }
}

template <int MB, int NB, int WM, int WN, int WK, int KG, int S, bool TAIL>
hipError_t launch_gemm32_f16_grid(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                                  int64_t n, int64_t k, int vec, hipStream_t stream) {
    using C = F16x32<MB, NB, WM, WN, WK, KG, S>;
    const int64_t tiles_n = (n + C::BN - 1) / C::BN;
    const int64_t tiles = tiles_n * ((m + C::BM - 1) / C::BM);
    static std::atomic<uint64_t> lds_done{0};
    hipError_t e = allow_dynamic_lds(
        reinterpret_cast<const void*>(&gemm32_f16_kernel<MB, NB, WM, WN, WK, KG, S, TAIL>),
        C::kLds, lds_done);
    if (e != hipSuccess) return e;
    for (int64_t base = 0; base < tiles; base += kGemmF16MaxGrid) {
        const int64_t grid = tiles - base < kGemmF16MaxGrid ? tiles - base : kGemmF16MaxGrid;
        hipLaunchKernelGGL((gemm32_f16_kernel<MB, NB, WM, WN, WK, KG, S, TAIL>),
                           dim3((unsigned)grid), dim3(C::kThreads), C::kLds, stream, x, w, y,
                           (int)m, n, (int)k, (int)(k / 32), tiles_n, base, vec);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int MB, int NB, int WM, int WN, int WK, int KG, int S>
hipError_t launch_gemm32_f16_t(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                               int64_t n, int64_t k, hipStream_t stream) {
    // 16-byte stores when every output row is 16-byte aligned
    const int vec = (reinterpret_cast<uintptr_t>(y) % 16) == 0 && n % 4 == 0;
    if ((k / 32) % KG != 0)
        return launch_gemm32_f16_grid<MB, NB, WM, WN, WK, KG, S, true>(x, w, y, m, n, k, vec,
                                                                       stream);
    return launch_gemm32_f16_grid<MB, NB, WM, WN, WK, KG, S, false>(x, w, y, m, n, k, vec,
                                                                    stream);
}

}  // namespace

hipError_t launch_gemm_f16(const uint16_t* x, const uint16_t* w, float* y, int64_t m,
                           int64_t n, int64_t k, hipStream_t stream) {
    if (m <= 8) return launch_gemv_f16(x, w, y, m, n, k, stream);
    if (m <= 16) return launch_gemm_f16_t<16, 1, 4, 2, 4>(x, w, y, m, n, k, stream);
    if (m <= 32) return launch_gemm_f16_t<32, 1, 4, 2, 4>(x, w, y, m, n, k, stream);
    // above, the 32 x 32 block kernel with the tile shape of least estimated
    // time (choose_tile).  Round times: one tile per CU, k = 2560, n = 4096,
    // measured on MI355X at m = 1024, 512, 256 and 128; they follow the
    // operand bytes a tile moves from L2 into LDS, (BM + BN) * k * 2, at
    // ~45-55 GB/s per CU.  For the 128 x 128 tile, 2-group stages in a
    // four-stage ring beat 4-group stages in two (m = 2048: 56.4-57.5 ->
    // 53.0-53.4 us); the other shapes were swept over ring depths of 2-6 and
    // 32 x 32 to 64 x 64 wave blocks without a gain.
    static constexpr TileChoice kTilesF16[] = {
        {128, 128, 27.7f},     // gemm32_f16_kernel<2, 2, 2, 2, 2, 2, 4>: 2 x 2 quadrants x 2 K phases
        {64, 128, 17.5f},      // gemm32_f16_kernel<2, 2, 1, 2, 4, 4, 3>: 2 column slices x 4 K phases
        {64, 64, 11.3f},       // gemm32_f16_kernel<2, 1, 1, 2, 4, 4, 4>
        {32, 64, 9.1f},        // gemm32_f16_kernel<1, 1, 1, 2, 4, 8, 3>
    };
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    switch (choose_tile(kTilesF16, 4, m, 1, &n, device_info(dev).cu_count)) {
        case 0: return launch_gemm32_f16_t<2, 2, 2, 2, 2, 2, 4>(x, w, y, m, n, k, stream);
        case 1: return launch_gemm32_f16_t<2, 2, 1, 2, 4, 4, 3>(x, w, y, m, n, k, stream);
        case 2: return launch_gemm32_f16_t<2, 1, 1, 2, 4, 4, 4>(x, w, y, m, n, k, stream);
        default: return launch_gemm32_f16_t<1, 1, 1, 2, 4, 8, 3>(x, w, y, m, n, k, stream);
    }
}

}  // namespace q4
