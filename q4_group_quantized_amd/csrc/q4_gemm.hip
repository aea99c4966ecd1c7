// q4_gemm.hip -- prefill Q4 product y = x * dequant(W)^T for many tokens on gfx950.
//
// Method: the batched prefill of the QORA pages, where every projection of a
// token batch is one matrix product over 4-bit weights (QORA-4B article, GPU
// prefill section; QORA-LLM-0.8B model card, "Performance"), with the Q4
// format of their quantization sections (symmetric, group size 32, 16-entry
// table dequantization).
//
// Arithmetic.  For every 32-element group j, one v_mfma_f32_16x16x32_f16 per
// 16x16 output block multiplies fp16 activations by the group's exact fp16
// levels -8..7 (K = 32 is exactly one group) into a fresh accumulator P, and
// the group's scale is applied in fp32 afterwards: acc += s[n, j] * P.  In the
// 16x16 D layout a lane's four values share one column, hence one scale.
//
// Work split.  A workgroup (4, 8 or 16 waves: one, two or four per SIMD) owns a
// BM x (16*NB*WN) tile of y (WN = 1, 2 or 4 column slices of NB = 1 or 2
// 16-column blocks).  Its waves are WN column slices x WK slices of K: each
// wave covers all BM rows and 16*NB columns over G/WK groups, so every code is
// unpacked by
// exactly one wave and every activation is read from LDS by WN waves.  The
// WK partial tiles are added in LDS at the end in a fixed order
// (deterministic).  The tile shape is chosen per launch from m and the number
// of tiles of all its matrices (choose_tile); the order of the fp32 sums, and
// so the last bits of a result, depend on that shape.
//
// Data movement.  Every operand goes straight from global memory into LDS
// with direct-to-LDS loads, through an S-stage ring per K slice:
//   activations  16 rows x 64 bytes of one group per wave instruction (1 KiB);
//                each lane reads its A operand with one ds_read_b128
//   codes        one whole 16-byte group of 64 columns per instruction
//                (two instructions per group for 128-column tiles; 32-column
//                tiles take two groups of their own 32 columns instead, so
//                no lane loads a neighbouring tile's codes)
//   scales       one fp16 per column, each landing in a 4-byte LDS slot
// so the loop body issues no register-destination global loads and the only
// waits on global memory are the explicit per-stage vmcnt waits below.
// Rows past M, columns past N and groups past G are clamped to real
// addresses: their results are never stored.  Groups past the end of a
// wave's K slice read zero activations and a zero scale from a block of LDS
// kept for that, so they add exactly 0 and the loop has no per-group branch.
#include "q4.h"
#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBlockBytes = 1024;          // one (group, 16-row block) of activations

__device__ __forceinline__ constexpr int vmcnt_imm(int n) {
    // s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 (gfx9)
    return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

template <int BM, int WN, int WK, int KG, int S, int NB = 2>
struct Gemm {
    static constexpr int MB = BM / 16;                     // 16-row blocks per wave
    static constexpr int BN = 16 * NB * WN;                        // NB 16-column blocks per wave
    static constexpr int H = (BN + 63) / 64;                         // 64-column code blocks
    // 16- and 32-column tiles load the codes and scales of 64 / BN groups per
    // instruction (lanes BN*j .. BN*j + BN-1 take group j of the block); 64-column
    // blocks take one group per instruction
    static constexpr bool kPair = BN < 64;
    static constexpr int kGPI = kPair ? 64 / BN : 1;                 // groups per code block
    static constexpr int kItems = kPair ? (KG + kGPI - 1) / kGPI : KG * H;   // per stage
    static constexpr int kCodeOff = KG * MB * kBlockBytes;           // within a stage
    static constexpr int kScaleOff = kCodeOff + kItems * kBlockBytes;
    static constexpr int kStageBytes = kScaleOff + kItems * 256;     // per K slice
    static constexpr int kABlocksPerWave = KG * MB / WN;
    // code block i of a stage (with its scales) is loaded by wave i % WN of
    // the K slice: group i / H, 64-column block i % H -- or, paired, groups
    // 2i and 2i + 1 of the tile's 32 columns
    static constexpr int groups_of(int wn) { return wn < WN ? (kItems - wn + WN - 1) / WN : 0; }
    static constexpr int loads_per_stage(int wn) { return kABlocksPerWave + 2 * groups_of(wn); }
    static constexpr int kLdsBytes = WK * S * kStageBytes;
    // zeros that the operand reads of out-of-range groups are pointed at
    static constexpr int kZeroBytes = MB * kBlockBytes;
    static constexpr int kLdsTotal = kLdsBytes + kZeroBytes;
    static constexpr int kRedBytes = (WK - 1) * WN * MB * NB * 4 * 64 * 4;
    static constexpr int kThreads = 64 * WN * WK;
    static_assert(WN * WK == 4 || WN * WK == 8 || WN * WK == 16, "one, two or four waves per SIMD");
    static_assert(WN <= 4 && H <= 2, "at most four column slices (128 columns)");
    static_assert((KG * MB) % WN == 0, "activation blocks split evenly");
    static_assert(S >= 2, "at least double buffering");
    static_assert(kRedBytes <= kLdsBytes, "reduction fits in the staging space");
    static_assert(kLdsTotal <= 160 * 1024, "LDS of one CU");
    static_assert(4 * BN <= kZeroBytes, "zero scale slots of every column");
};

// The matrices of one launch: up to kGemmMaxSegments weight matrices over the
// same activations (one for q4_gemm).  Segment s owns workgroups
// [tile0[s], tile0[s] + tiles[s]); a tile's work and its order of fp32 sums
// depend only on its index inside its segment and on the launch's tile shape,
// never on the other matrices of the launch.
constexpr int kGemmMaxSegments = 8;
// Workgroups per launch at most: the dispatch counts work-items in 32 bits, and
// 2^20 workgroups of up to 1024 threads stay below that.  Larger tile counts
// take several launches, each starting at its own first tile.
constexpr int64_t kGemmMaxGrid = 1 << 20;
struct GemmSegments {
    const uint8_t* packed[kGemmMaxSegments];
    const uint16_t* scales[kGemmMaxSegments];
    float* y[kGemmMaxSegments];
    int64_t n[kGemmMaxSegments];
    int64_t tiles_n[kGemmMaxSegments];
    int64_t tile0[kGemmMaxSegments];
    int count;
};
static_assert(kGemmMaxSegments == Q4_MULTI_MAX, "segment table must hold Q4_MULTI_MAX matrices");

// At least two waves per SIMD: caps a wave at 256 registers (128 for the
// 16-wave workgroups, which need four per SIMD), which also makes the compiler
// keep MFMA results in VGPRs instead of routing them through AGPRs (four
// v_accvgpr_read per 16x16 block before the scale FMAs).
template <int BM, int WN, int WK, int KG, int S, int NB>
__global__ __launch_bounds__(64 * WN * WK, 2) void gemm_kernel(
    const uint16_t* __restrict__ x, GemmSegments seg, int M, int K, int G, SpliceConsts kc,
    int64_t tile_base) {
    using C = Gemm<BM, WN, WK, KG, S, NB>;
    constexpr int MB = C::MB;
    extern __shared__ __align__(16) unsigned char smem[];

    // this workgroup's matrix (selects over constant indices, workgroup-uniform)
    const uint8_t* packed = seg.packed[0];
    const uint16_t* scales = seg.scales[0];
    float* y = seg.y[0];
    int64_t N = seg.n[0], tiles_n = seg.tiles_n[0], tile0 = seg.tile0[0];
    const int64_t gt = tile_base + blockIdx.x;           // tile over all segments
#pragma unroll
    for (int i = 1; i < kGemmMaxSegments; ++i) {
        if (i < seg.count && gt >= seg.tile0[i]) {
            packed = seg.packed[i]; scales = seg.scales[i]; y = seg.y[i];
            N = seg.n[i]; tiles_n = seg.tiles_n[i]; tile0 = seg.tile0[i];
        }
    }
    const int64_t tile = gt - tile0;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar branches
    const int wn = wave % WN;
    const int kp = wave / WN;
    const int64_t nt0 = (tile % tiles_n) * C::BN;     // tile's first column
    const int64_t m0 = (tile / tiles_n) * BM;

    const int Gp = (G + WK - 1) / WK;                     // groups per K slice
    const int gbeg = kp * Gp;
    const int gend = min(G, gbeg + Gp);
    const int nstages = (Gp + KG - 1) / KG;               // same for every wave

    unsigned char* kbase = smem + (size_t)kp * S * C::kStageBytes;
    // A group past the slice's end (the last stage of a slice whose group
    // count is not a multiple of KG) reads its activations and scale from
    // this zero block: its MFMA then gives exactly 0 (levels are finite) and
    // its scale FMA adds 0 * 0, so every group is computed without a branch.
    const unsigned char* zero = smem + C::kLdsBytes;
    for (int i = threadIdx.x; i < C::kZeroBytes / 16; i += C::kThreads)
        reinterpret_cast<u32x4_t*>(smem + C::kLdsBytes)[i] = u32x4_t{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0): zeros stored before the first barrier
    // Workgroups start their walk over K at a stage set by their column tile:
    // tiles of different columns spread their requests for the same activation
    // rows over K, while the row tiles of one column (on one XCD when the
    // number of column tiles is a multiple of 8) walk its weights in step and
    // share them in L2.  The order of
    // the fp32 sums depends only on the tile index, identically on every run.
    const int rot = (int)((tile % tiles_n) % nstages);
    auto stage_group = [&](int st) {               // first group (in the slice) of stage st
        const int r = st + rot;
        return (r < nstages ? r : r - nstages) * KG;
    };

    // load-side lane mappings
    const int a_row = lane >> 2, a_part = lane & 3;       // 16 rows x 4 16-byte parts
    // codes / scales: lane = column of a 64-column block (two scalar pointers:
    // a local array of pointers here made the compiler drop the kernel's host stub)
    const int64_t ld_col0 = min<int64_t>(nt0 + lane, N - 1);
    const int64_t ld_col1 = min<int64_t>(nt0 + 64 + lane, N - 1);
    const uint8_t* code_row0 = packed + ld_col0 * (K / 2);
    const uint8_t* code_row1 = packed + ld_col1 * (K / 2);
    const uint16_t* scale_row0 = scales + ld_col0 * G;
    const uint16_t* scale_row1 = scales + ld_col1 * G;
    // paired layout: lane = column (lane % 32) of group 2i + lane / 32
    const int64_t pr_col = min<int64_t>(nt0 + lane % C::BN, N - 1);
    const uint8_t* code_rowp = packed + pr_col * (K / 2);
    const uint16_t* scale_rowp = scales + pr_col * G;
    const int pr_g = lane / C::BN;
    // operand-side lane mapping
    const int col = lane & 15, kq = lane >> 4;

    auto issue = [&](int st, int buf) {
        unsigned char* sb = kbase + buf * C::kStageBytes;
        const int gs = gbeg + stage_group(st);
#pragma unroll
        for (int i = 0; i < C::kABlocksPerWave; ++i) {
            const int b = wn * C::kABlocksPerWave + i;
            const int gl = b / MB, mb = b % MB;
            const int g = min(gs + gl, G - 1);
            const int64_t r = min<int64_t>(m0 + 16 * mb + a_row, M - 1);
            __builtin_amdgcn_global_load_lds(x + r * K + 32 * g + 8 * a_part,
                                             (lds_void_t*)(sb + (gl * MB + mb) * kBlockBytes),
                                             16, 0, 0);
        }
        if constexpr (C::kPair) {
#pragma unroll
            for (int it = 0; it < C::kItems; ++it) {
                const int g = min(gs + C::kGPI * it + pr_g, G - 1);
                __builtin_amdgcn_global_load_lds(code_rowp + 16 * g,
                                                 (lds_void_t*)(sb + C::kCodeOff + it * kBlockBytes),
                                                 16, 0, 0);
                __builtin_amdgcn_global_load_lds(scale_rowp + g,
                                                 (lds_void_t*)(sb + C::kScaleOff + it * 256), 2,
                                                 0, 0);
            }
            return;
        }
#pragma unroll
        for (int it = 0; it < KG * C::H; ++it) {
            if (it % WN != wn) continue;
            const int gl = it / C::H, h = it % C::H;
            const int g = min(gs + gl, G - 1);
            __builtin_amdgcn_global_load_lds((h ? code_row1 : code_row0) + 16 * g,
                                             (lds_void_t*)(sb + C::kCodeOff + it * kBlockBytes),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((h ? scale_row1 : scale_row0) + g,
                                             (lds_void_t*)(sb + C::kScaleOff + it * 256), 2, 0,
                                             0);
        }
    };

    float4_t acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t mask = kc.mask;
    const uint32_t magic = to_vgpr(kc.magic);
    const uint32_t sel[4] = {kc.sel[0], kc.sel[1], kc.sel[2], kc.sel[3]};

#pragma unroll
    for (int u = 0; u < S - 1; ++u) issue(u, u);

    // Operands of one group, read from LDS ahead of use: while a group's
    // MFMAs and scale FMAs run, the next group's reads are in flight.
    struct Ops {
        half8_t a[MB];
        uint32_t code[NB];
        _Float16 sc[NB];
    };
    auto read_ops = [&](Ops& o, const unsigned char* sb, int gl, bool valid) {
        const unsigned char* ab = valid ? sb + gl * MB * kBlockBytes : zero;
        const int item = C::kPair ? gl / C::kGPI : gl * C::H;       // first code block of group gl
        const int e0 = C::kPair ? C::BN * (gl % C::kGPI) : 0;         // its first entry there
        const unsigned char* scb = valid ? sb + C::kScaleOff + item * 256 : zero;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            o.a[mb] = *reinterpret_cast<const half8_t*>(ab + mb * kBlockBytes + 64 * col + 16 * kq);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int c = 16 * NB * wn + 16 * nb + col;
            o.code[nb] = *reinterpret_cast<const uint32_t*>(
                sb + C::kCodeOff + item * kBlockBytes + 16 * (e0 + c) + 4 * kq);
            o.sc[nb] = *reinterpret_cast<const _Float16*>(scb + 4 * (e0 + c));
        }
    };
    auto compute = [&](const Ops& o) {
        half8_t bh[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) bh[nb] = unpack8_natural(o.code[nb], mask, magic, sel);
        // all MFMAs of the group first, so their latencies overlap, then the
        // scale FMAs
        float4_t p[MB][NB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float4_t zero = {0.f, 0.f, 0.f, 0.f};
                p[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.a[mb], bh[nb], zero, 0, 0, 0);
            }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float s = (float)o.sc[nb];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[mb][nb][v] = fmaf(s, p[mb][nb][v], acc[mb][nb][v]);
        }
    };

    for (int st0 = 0; st0 < nstages; st0 += S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            const int st = st0 + u;
            if (st < nstages) {
                // stage st has landed once at most the S-2 later stages remain in
                // flight (wave-uniform branch: the count depends on the wave's share)
                if (WN == 1 || wn == 0)
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::loads_per_stage(0) * (S - 2)));
                else if (wn == 1)
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::loads_per_stage(1) * (S - 2)));
                else if (wn == 2)
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::loads_per_stage(2) * (S - 2)));
                else
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::loads_per_stage(3) * (S - 2)));
                barrier_keep_loads();
                // refill the buffer computed last iteration (every wave is past it)
                issue(st + S - 1, (u + S - 1) % S);
                const unsigned char* sb = kbase + u * C::kStageBytes;
                const int g0 = gbeg + stage_group(st);
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
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    if (kp > 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    red[((((kp - 1) * WN + wn) * MB + mb) * NB * 4 + nb * 4 + v) * 64 + lane] =
                        acc[mb][nb][v];
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int64_t n = nt0 + 16 * NB * wn + 16 * nb + col;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float t = acc[mb][nb][v];
#pragma unroll
                    for (int q = 1; q < WK; ++q)
                        t += red[((((q - 1) * WN + wn) * MB + mb) * NB * 4 + nb * 4 + v) * 64 + lane];
                    const int64_t m = m0 + 16 * mb + 4 * kq + v;
                    if (m < M && n < N) y[m * N + n] = t;
                }
            }
    }
}

template <int BM, int WN, int WK, int KG, int S, int NB = 2>
hipError_t launch_gemm_t(const uint16_t* x, int count, const uint8_t* const* packed,
                         const uint16_t* const* scales, float* const* y, const int64_t* n,
                         int64_t m, int64_t k, hipStream_t stream) {
    using C = Gemm<BM, WN, WK, KG, S, NB>;
    GemmSegments seg = {};
    seg.count = count;
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
        seg.packed[i] = packed[i];
        seg.scales[i] = scales[i];
        seg.y[i] = y[i];
        seg.n[i] = n[i];
        seg.tiles_n[i] = (n[i] + C::BN - 1) / C::BN;
        seg.tile0[i] = tiles;
        tiles += seg.tiles_n[i] * ((m + BM - 1) / BM);
    }
    static std::atomic<uint64_t> lds_done{0};           // devices already set up
    hipError_t e = allow_dynamic_lds(
        reinterpret_cast<const void*>(&gemm_kernel<BM, WN, WK, KG, S, NB>), C::kLdsTotal, lds_done);
    if (e != hipSuccess) return e;
    for (int64_t base = 0; base < tiles; base += kGemmMaxGrid) {
        const int64_t grid = tiles - base < kGemmMaxGrid ? tiles - base : kGemmMaxGrid;
        hipLaunchKernelGGL((gemm_kernel<BM, WN, WK, KG, S, NB>), dim3((unsigned)grid),
                           dim3(C::kThreads), C::kLdsTotal, stream, x, seg, (int)m, (int)k,
                           (int)(k / 32), kSpliceConsts, base);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Tile shapes for m > 32, largest first, with the time one full round of
// them takes (k = 2560, n = 4096, one tile per CU; measured).
constexpr TileChoice kTiles[] = {
    {128, 128, 35.f},      // gemm_kernel<128, 4, 2, 2, 2>
    {64, 128, 22.f},       // gemm_kernel<64, 4, 4, 2, 2> (16 waves)
    {64, 64, 15.5f},       // gemm_kernel<64, 2, 4, 2, 2>
    {32, 64, 11.f},        // gemm_kernel<32, 2, 4, 2, 2>
};

hipError_t launch_gemm_segments(const uint16_t* x, int count, const uint8_t* const* packed,
                                const uint16_t* const* scales, float* const* y,
                                const int64_t* n, int64_t m, int64_t k, hipStream_t stream) {
    if (m <= 16)      // 16 x 16 tiles: the weight traffic of a small batch spread over every CU
        return launch_gemm_t<16, 1, 4, 4, 4, 1>(x, count, packed, scales, y, n, m, k, stream);
    if (m <= 32)      // 32 x 16 tiles (measured 10.5 -> 8.0 us at m = 32, n = 4096, k = 2560)
        return launch_gemm_t<32, 1, 4, 4, 3, 1>(x, count, packed, scales, y, n, m, k, stream);
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    switch (choose_tile(kTiles, 4, m, count, n, device_info(dev).cu_count)) {
        case 0: return launch_gemm_t<128, 4, 2, 2, 2>(x, count, packed, scales, y, n, m, k, stream);
        case 1: return launch_gemm_t<64, 4, 4, 2, 2>(x, count, packed, scales, y, n, m, k, stream);
        case 2: return launch_gemm_t<64, 2, 4, 2, 2>(x, count, packed, scales, y, n, m, k, stream);
        default: return launch_gemm_t<32, 2, 4, 2, 2>(x, count, packed, scales, y, n, m, k, stream);
    }
}

}  // namespace

hipError_t launch_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                       float* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
    if (m <= 8) return launch_gemv(x, packed, scales, y, m, n, k, stream);
    return launch_gemm_segments(x, 1, &packed, &scales, &y, &n, m, k, stream);
}

hipError_t launch_gemm_multi(const uint16_t* x, int64_t m, int64_t k, int count,
                             const uint8_t* const* packed, const uint16_t* const* scales,
                             float* const* y, const int64_t* n, hipStream_t stream) {
    if (m <= 8) return launch_gemv_multi(x, m, k, count, packed, scales, y, n, stream);
    return launch_gemm_segments(x, count, packed, scales, y, n, m, k, stream);
}

}  // namespace q4
