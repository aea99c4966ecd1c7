// q4_gemm.hip -- prefill Q4 product y = x * dequant(W)^T for many tokens on gfx950.
//
// Method: the batched prefill of the QORA pages, where every projection of a
// token batch is one matrix product over 4-bit weights (QORA-4B article, GPU
// prefill section; QORA-LLM-0.8B model card, "Performance"), with the Q4
// format of their quantization sections (symmetric, group size 32, 16-entry
// table dequantization).
//
// Two kernels.  m <= 32 runs gemm_kernel below (16 x 16 output blocks,
// 16- or 32-row tiles of 16 columns, so a small batch still spreads its
// weight traffic over every CU); m > 32 runs gemm32_kernel further down
// (32 x 32 output blocks, tiles of 32 x 64 up to 128 x 128 chosen per launch).
// Both apply each group's scale in fp32 after that group's own MFMA.
//
// Arithmetic (gemm_kernel).  For every 32-element group j, one
// v_mfma_f32_16x16x32_f16 per 16x16 output block multiplies fp16 activations by
// the group's exact fp16 levels -8..7 (K = 32 is exactly one group) into a
// fresh accumulator P, and the group's scale is applied in fp32 afterwards:
// acc += s[n, j] * P.  In the 16x16 D layout a lane's four values share one
// column, hence one scale.
//
// Work split.  A workgroup (4, 8 or 16 waves: one, two or four per SIMD) owns a
// BM x (16*NB*WN) tile of y (WN = 1, 2 or 4 column slices of NB = 1 or 2
// 16-column blocks).  Its waves are WN column slices x WK slices of K: each
// wave covers all BM rows and 16*NB columns over G/WK groups, so every code is
// unpacked by
// exactly one wave and every activation is read from LDS by WN waves.  The
// WK partial tiles are added in LDS at the end in a fixed order
// (deterministic).  The tile shape (for m > 32, gemm32_kernel's) is chosen
// per launch from m and the number of tiles of all its matrices
// (choose_tile); the order of the fp32 sums, and so the last bits of a
// result, depend on that shape.
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
                // With one column slice (WN = 1) every wave loads and reads only
                // its own K slice's ring, so after the first stage (which also
                // publishes the zero block) the waves need no common barrier
                // and run apart (m = 8 / 16 at k = 2560: 3-4% faster, same bits).
                if (WN > 1 || st == 0) barrier_keep_loads();
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

// ---------------------------------------------------------------------------
// m > 32: 32 x 32 output blocks (v_mfma_f32_32x32x16_f16)
//
// Per 32-element group and 32 x 32 block: two MFMAs (K = 16 each) into a
// fresh P, then acc += s * P, where a lane's 16 values of the 32 x 32 D
// layout share one column (lane % 32) and hence one scale.  Per MAC this
// issues half the MFMA instructions of 16 x 16 blocks; the sixteen fp32 scale
// FMAs per block and group are the same count either way.
//
// Work split.  A workgroup of WN x WK waves owns a BM x BN tile of y (BM =
// 32 MB rows, BN = 32 NB WN columns).  Wave (wn, wk) computes all BM rows of
// columns [32 NB wn, 32 NB (wn + 1)) over the groups wk, wk + WK, ... of
// every stage, so a code is unpacked once per workgroup and shared by the MB
// row blocks.  The WK partial tiles are added in LDS in a fixed order.
//
// Data movement.  A stage holds KG consecutive groups of the tile: every
// operand goes global -> LDS with direct loads, each wave instruction
// reading whole rows of the stage (activations: 64/(4 KG) rows x 64 KG
// bytes; codes: 64/KG columns x 16 KG bytes; scales: 64 of them, 2 bytes
// each into 4-byte slots).  LDS layouts are XOR-swizzled so that the
// operand reads of a wave touch distinct banks: activation chunk c (16 B)
// of tile row r sits at position c ^ (r & 7) of the row, code group gl of
// column j at position gl ^ ((j >> 1) & (KG - 1)).  The loads choose their
// global addresses to fill those positions, so the loop reads LDS at fixed
// per-lane offsets and issues no address arithmetic per operand.
// K mapping inside a group: lane (i, g) (i = lane % 32, g = lane / 32) feeds
// the MFMA h (h = 0, 1) with the 8 elements of chunk 2g + h, for the
// activation row i and for the code column i alike.
// ---------------------------------------------------------------------------
typedef float float16v_t __attribute__((ext_vector_type(16)));
// Per-lane load offsets are kept in a vector type: with a plain local array
// in the address of a direct-to-LDS load the host compiler drops the
// kernel's launch stub.
typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));

template <int MB, int NB, int WN, int WK, int KG, int S, bool SV>
struct G32 {
    static constexpr int BM = 32 * MB;
    static constexpr int BN = 32 * NB * WN;
    static constexpr int W = WN * WK;
    static constexpr int kThreads = 64 * W;
    static constexpr int GPW = KG / WK;                  // groups per wave and stage
    static constexpr int kRowBytes = KG * 64;            // activations of one row
    static constexpr int kColBytes = KG * 16;            // codes of one column
    static constexpr int kABytes = BM * kRowBytes;
    static constexpr int kCBytes = BN * kColBytes;
    // scales: SV (4-byte loads of two groups): [column][KG groups] fp16;
    // else one 2-byte load per (group, column) into 4-byte slots,
    // [group][column]
    static constexpr int kSBytes = SV ? BN * KG * 2 : KG * BN * 4;
    static constexpr int kStage = kABytes + kCBytes + kSBytes;
    static constexpr int NA = kABytes / 1024;            // load instructions per stage
    static constexpr int NC = kCBytes / 1024;
    static constexpr int NS = SV ? BN * KG / 128 : KG * BN / 64;
    static constexpr int NAW = NA / W, NCW = NC / W, NSW = NS / W;
    static constexpr int kLoadsPerWave = NAW + NCW + NSW;
    // the WK partial tiles, row-major with rows of RS floats
    static constexpr int RS = BN + 4;
    static constexpr int kRedBytes = WK * BM * RS * 4;
    static constexpr int kLds = S * kStage > kRedBytes ? S * kStage : kRedBytes;
    static constexpr int CPR = 4 * KG;                   // 16-byte chunks per activation row
    static constexpr int RPI = 64 / CPR;                 // rows per load instruction
    static constexpr int CPI = 64 / KG;                  // code columns per load instruction
    static_assert(KG % WK == 0, "whole groups per wave");
    static_assert(KG == 2 || KG == 4 || KG == 8 || KG == 16, "power-of-two stage");
    static_assert(!SV || KG % 2 == 0, "4-byte scale loads hold two groups");
    static_assert(NA % W == 0 && NC % W == 0 && NS % W == 0, "equal loads per wave");
    static_assert(W == 4 || W == 8 || W == 16, "one, two or four waves per SIMD");
    static_assert(NAW <= 16 && NCW <= 16 && NSW <= 16, "load offsets fit one u32x16_t");
    static_assert(S >= 2, "at least double buffering");
    static_assert(kLds <= 160 * 1024, "LDS of one CU");
    // a stage issues the next stage's loads after its second block
    static_assert(MB * NB >= 2, "at least two 32x32 blocks per wave");
};

template <int MB, int NB, int WN, int WK, int KG, int S, bool SV, bool TAIL>
__global__ __launch_bounds__(64 * WN * WK, 1) void gemm32_kernel(
    const uint16_t* __restrict__ x, GemmSegments seg, int M, int K, int G, SpliceConsts kc,
    int64_t tile_base, int vec_store) {
    using C = G32<MB, NB, WN, WK, KG, S, SV>;
    extern __shared__ __align__(16) unsigned char smem[];

    const uint8_t* packed = seg.packed[0];
    const uint16_t* scales = seg.scales[0];
    float* y = seg.y[0];
    int64_t N = seg.n[0], tiles_n = seg.tiles_n[0], tile0 = seg.tile0[0];
    const int64_t gt = tile_base + blockIdx.x;
#pragma unroll
    for (int i = 1; i < kGemmMaxSegments; ++i) {
        if (i < seg.count && gt >= seg.tile0[i]) {
            packed = seg.packed[i]; scales = seg.scales[i]; y = seg.y[i];
            N = seg.n[i]; tiles_n = seg.tiles_n[i]; tile0 = seg.tile0[i];
        }
    }
    const int64_t tile = gt - tile0;
    const int64_t n0 = (tile % tiles_n) * C::BN;
    const int64_t m0 = (tile / tiles_n) * C::BM;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % WN, wk = wave / WN;
    const int li = lane & 31, lg = lane >> 5;
    const int nstages = (G + KG - 1) / KG;

    // ---- per-lane load offsets (bytes from the stage's uniform bases) ----
    u32x16_t offA = {}, offC = {}, offS = {};
    int ldsA[C::NAW], ldsC[C::NCW], ldsS[C::NSW];
    int grpA[C::NAW], grpC[C::NCW], grpS[C::NSW];   // group of the stage each lane loads
#pragma unroll
    for (int t = 0; t < C::NAW; ++t) {
        const int q = wave * C::NAW + t;
        const int r = q * C::RPI + lane / C::CPR;
        const int c = (lane % C::CPR) ^ (r & 7);
        const int64_t row = min<int64_t>(m0 + r, M - 1) - m0;
        grpA[t] = c >> 2;
        offA[t] = (uint32_t)(row * K * 2) + (uint32_t)(c * 16);
        ldsA[t] = q * 1024;
    }
#pragma unroll
    for (int t = 0; t < C::NCW; ++t) {
        const int q = wave * C::NCW + t;
        const int j = q * C::CPI + lane / KG;
        const int gl = (lane % KG) ^ ((j >> 1) & (KG - 1));
        const int64_t col = min<int64_t>(n0 + j, N - 1) - n0;
        grpC[t] = gl;
        offC[t] = (uint32_t)(col * (K / 2)) + (uint32_t)(gl * 16);
        ldsC[t] = C::kABytes + q * 1024;
    }
#pragma unroll
    for (int t = 0; t < C::NSW; ++t) {
        const int q = wave * C::NSW + t;
        if (SV) {              // lane: column j, groups 2d and 2d + 1 of the stage
            const int piece = q * 64 + lane;
            const int j = piece / (KG / 2), d = piece % (KG / 2);
            const int64_t col = min<int64_t>(n0 + j, N - 1) - n0;
            grpS[t] = 2 * d;
            offS[t] = (uint32_t)((col * G + 2 * d) * 2);
            ldsS[t] = C::kABytes + C::kCBytes + q * 256;
        } else {
            const int slot = q * 64 + lane;
            const int gl = slot / C::BN, j = slot % C::BN;
            const int64_t col = min<int64_t>(n0 + j, N - 1) - n0;
            grpS[t] = gl;
            offS[t] = (uint32_t)((col * G + gl) * 2);
            ldsS[t] = C::kABytes + C::kCBytes + q * 256;
        }
    }
    const unsigned char* xbase = reinterpret_cast<const unsigned char*>(x + m0 * K);
    const unsigned char* cbase = packed + n0 * (K / 2);
    const unsigned char* sbase = reinterpret_cast<const unsigned char*>(scales + n0 * G);

    // Loads of stage st into ring buffer buf.  With TAIL (G not a multiple
    // of KG), groups past G in the last stage re-read group G - 1 (in bounds;
    // their results are not used): the step back is a per-lane select, so the
    // loop has no branch here.
    auto issue = [&](int st, int buf) {
        unsigned char* sb = smem + buf * C::kStage;
        const int g0 = st * KG;
        const int over = g0 - (G - 1);                    // > -KG only in the last stage
        auto step_back = [&](int grp, uint32_t unit) {
            return TAIL ? (uint32_t)max(0, over + grp) * unit : 0u;
        };
#pragma unroll
        for (int t = 0; t < C::NAW; ++t) {
            const uint32_t back = step_back((int)grpA[t], 64u);
            __builtin_amdgcn_global_load_lds(xbase + (size_t)g0 * 64 + (offA[t] - back),
                                             (lds_void_t*)(sb + ldsA[t]), 16, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < C::NCW; ++t) {
            const uint32_t back = step_back((int)grpC[t], 16u);
            __builtin_amdgcn_global_load_lds(cbase + (size_t)g0 * 16 + (offC[t] - back),
                                             (lds_void_t*)(sb + ldsC[t]), 16, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < C::NSW; ++t) {
            if (SV) {
                // G is even here, so a pair never straddles G
                const uint32_t back = step_back((int)grpS[t], 2u);
                __builtin_amdgcn_global_load_lds(sbase + (size_t)g0 * 2 + (offS[t] - back),
                                                 (lds_void_t*)(sb + ldsS[t]), 4, 0, 0);
            } else {
                const uint32_t back = step_back((int)grpS[t], 2u);
                __builtin_amdgcn_global_load_lds(sbase + (size_t)g0 * 2 + (offS[t] - back),
                                                 (lds_void_t*)(sb + ldsS[t]), 2, 0, 0);
            }
        }
    };

    // ---- per-lane operand offsets inside a stage ----
    int rA[C::GPW][2], rC[C::GPW], rS[C::GPW];
#pragma unroll
    for (int u = 0; u < C::GPW; ++u) {
        const int gl = wk + WK * u;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            rA[u][h] = li * C::kRowBytes + (((gl * 4 + 2 * lg + h) ^ (li & 7)) * 16);
        const int j = 32 * NB * wn + li;
        rC[u] = C::kABytes + j * C::kColBytes + ((gl ^ ((li >> 1) & (KG - 1))) * 16) + 8 * lg;
        rS[u] = C::kABytes + C::kCBytes + (SV ? (j * KG + gl) * 2 : (gl * C::BN + j) * 4);
    }

    float16v_t acc[MB][NB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rb][nb][v] = 0.f;

    const uint32_t mask = kc.mask;
    const uint32_t magic = to_vgpr(kc.magic);
    const uint32_t sel[4] = {kc.sel[0], kc.sel[1], kc.sel[2], kc.sel[3]};

    // Operands of group u of this wave from stage buffer sb: activations of
    // the MB row blocks, unpacked levels of the NB column blocks, scales.
    struct Ops {
        half8_t a[MB][2];
        half8_t b[NB][2];
        float s[NB];
    };
    auto read_ops = [&](Ops& o, uint32_t (&cd)[NB][2], const unsigned char* sb, int u) {
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                o.a[rb][h] =
                    *reinterpret_cast<const half8_t*>(sb + rA[u][h] + rb * 32 * C::kRowBytes);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint2 c2 = *reinterpret_cast<const uint2*>(sb + rC[u] + nb * 32 * C::kColBytes);
            cd[nb][0] = c2.x;
            cd[nb][1] = c2.y;
            // widened once and passed through an identity DPP move: the FMAs
            // below then take a plain fp32 operand (v_fmac_f32) instead of
            // converting the fp16 scale inside each one (v_fma_mix_f32, ~13%
            // slower)
            const float sf =
                (float)*reinterpret_cast<const _Float16*>(sb + rS[u] + nb * (SV ? 64 * KG : 128));
            o.s[nb] = __builtin_bit_cast(
                float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sf), 0xE4, 0xF, 0xF, false));
        }
    };
    auto unpack_ops = [&](Ops& o, const uint32_t (&cd)[NB][2]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int h = 0; h < 2; ++h) o.b[nb][h] = unpack8_natural(cd[nb][h], mask, magic, sel);
    };
    auto mfma2 = [&](const Ops& o, int rb, int nb) {
        const float16v_t zero = {};
        float16v_t p = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.a[rb][0], o.b[nb][0], zero, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(o.a[rb][1], o.b[nb][1], p, 0, 0, 0);
    };
    auto scale_add = [&](float16v_t& dst, float s, const float16v_t& p) {
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[v] = fmaf(s, p[v], dst[v]);
    };

    // One stage, software-pipelined: the MFMAs of a block are issued before
    // the scale FMAs of the block before it, so the matrix core and the VALU
    // work at once within the wave.  The last block's product (pc, scale sc,
    // destination acc[MB - 1][NB - 1]) is carried into the next stage.
    // The loads of a later stage (nxt into ring buffer nbuf) are issued after
    // the first block, so their issue overlaps compute instead of every wave
    // queueing its loads at once right after the barrier.
    auto stage = [&](const unsigned char* sb, float16v_t& pc, float& sc, int nxt, int nbuf) {
        Ops ops[2];
        uint32_t cd[2][NB][2];
        read_ops(ops[0], cd[0], sb, 0);
        unpack_ops(ops[0], cd[0]);
#pragma unroll
        for (int u = 0; u < C::GPW; ++u) {
            Ops& o = ops[u & 1];
            if (u + 1 < C::GPW) read_ops(ops[(u + 1) & 1], cd[(u + 1) & 1], sb, u + 1);
#pragma unroll
            for (int rb = 0; rb < MB; ++rb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if (u == 0 && rb * NB + nb == 1) issue(nxt, nbuf);
                    const float16v_t p = mfma2(o, rb, nb);
                    // the block before this one, at raised wave priority: while
                    // one wave of a SIMD runs its scale FMAs the other's MFMAs
                    // queue behind them rather than the reverse (M = 512 19.2
                    // -> 18.6 us; other shapes within 1%)
                    __builtin_amdgcn_s_setprio(1);
                    const int prev = rb * NB + nb - 1;
                    if (prev < 0)
                        scale_add(acc[MB - 1][NB - 1], sc, pc);
                    else
                        scale_add(acc[prev / NB][prev % NB], o.s[prev % NB], pc);
                    __builtin_amdgcn_s_setprio(0);
                    pc = p;
                    // keep this order: left alone the scheduler hoists every
                    // MFMA of the unrolled stages ahead of the FMAs, holding
                    // many products in registers at once
                    __builtin_amdgcn_sched_barrier(0);
                }
            sc = o.s[NB - 1];
            if (u + 1 < C::GPW) unpack_ops(ops[(u + 1) & 1], cd[(u + 1) & 1]);
        }
    };

    // one group u of this wave, not pipelined (last stages)
    auto group = [&](const unsigned char* sb, int u) {
        Ops o;
        uint32_t cd[NB][2];
        read_ops(o, cd, sb, u);
        unpack_ops(o, cd);
#pragma unroll
        for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) scale_add(acc[rb][nb], o.s[nb], mfma2(o, rb, nb));
    };

    // Every iteration issues one stage's loads (stages past the end re-load
    // the last one into a buffer nobody reads again), so stage st has landed
    // once at most S - 2 later stages' loads remain in flight; after the
    // barrier every wave's loads of it have landed, and every wave is done
    // with the buffer that the refill overwrites.
    auto wait_stage = [&]() {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::kLoadsPerWave * (S - 2)));
        barrier_keep_loads();
    };

#pragma unroll
    for (int u = 0; u < S - 1; ++u) issue(min(u, nstages - 1), u);

    // full stages, S at a time (ring buffers at fixed offsets, no branch
    // inside, so the pipelined order above holds)
    const int nfull = G / KG;
    int st = 0;
    float16v_t pc = {};
    float sc = 0.f;
    for (; st + S <= nfull; st += S) {
#pragma unroll
        for (int b = 0; b < S; ++b) {
            wait_stage();
            stage(smem + b * C::kStage, pc, sc, min(st + b + S - 1, nstages - 1), (b + S - 1) % S);
        }
    }
    // the other full stages (fewer than S)
    for (; st < nfull; ++st) {
        const int b = st % S;
        wait_stage();
        stage(smem + b * C::kStage, pc, sc, min(st + S - 1, nstages - 1), (b + S - 1) % S);
    }
    scale_add(acc[MB - 1][NB - 1], sc, pc);
    // a partial last stage (G not a multiple of KG)
    if (nfull < nstages) {
        const int b = nfull % S;
        wait_stage();
        const unsigned char* sb = smem + b * C::kStage;
#pragma unroll
        for (int u = 0; u < C::GPW; ++u)
            if (nfull * KG + wk + WK * u < G) group(sb, u);
    }

    // ---- add the WK partial tiles (fixed order) and store ----
    // Every wave parks its partial tile row-major in LDS (partial wk at
    // red + wk * BM * RS, rows padded to RS floats so the two lane halves of
    // a write hit different banks); then every thread adds the WK partials of
    // its 4-float pieces in phase order 0, 1, ..., WK - 1 and stores them, 16
    // bytes per lane where the rows allow.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    {
        float* dst = red + wk * C::BM * C::RS + 32 * NB * wn + li;
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
    // row-major tile: BM rows x BN / 4 four-float pieces
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

template <int MB, int NB, int WN, int WK, int KG, int S, bool SV, bool TAIL>
hipError_t launch_gemm32_grid(const uint16_t* x, const GemmSegments& seg, int64_t tiles,
                              int64_t m, int64_t k, int vec, hipStream_t stream) {
    using C = G32<MB, NB, WN, WK, KG, S, SV>;
    static std::atomic<uint64_t> lds_done{0};
    hipError_t e = allow_dynamic_lds(
        reinterpret_cast<const void*>(&gemm32_kernel<MB, NB, WN, WK, KG, S, SV, TAIL>), C::kLds,
        lds_done);
    if (e != hipSuccess) return e;
    for (int64_t base = 0; base < tiles; base += kGemmMaxGrid) {
        const int64_t grid = tiles - base < kGemmMaxGrid ? tiles - base : kGemmMaxGrid;
        hipLaunchKernelGGL((gemm32_kernel<MB, NB, WN, WK, KG, S, SV, TAIL>), dim3((unsigned)grid),
                           dim3(C::kThreads), C::kLds, stream, x, seg, (int)m, (int)k,
                           (int)(k / 32), kSpliceConsts, base, vec);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// whether the 4-byte scale loads split evenly over the waves of a shape
template <int MB, int NB, int WN, int WK, int KG, int S>
struct SvOk {
    static constexpr bool value = KG % 2 == 0 && (32 * NB * WN * KG / 128) % (WN * WK) == 0;
};

template <int MB, int NB, int WN, int WK, int KG, int S>
hipError_t launch_gemm32_t(const uint16_t* x, int count, const uint8_t* const* packed,
                           const uint16_t* const* scales, float* const* y, const int64_t* n,
                           int64_t m, int64_t k, hipStream_t stream) {
    GemmSegments seg = {};
    seg.count = count;
    int64_t tiles = 0;
    constexpr int BM = 32 * MB, BN = 32 * NB * WN;
    // 4-byte scale loads (two groups per lane): every pair 4-byte aligned, and
    // as many of them per stage as there are waves
    bool sv = SvOk<MB, NB, WN, WK, KG, S>::value && (k / 32) % 2 == 0;
    // 16-byte stores: every row of every output 16-byte aligned
    int vec = 1;
    for (int i = 0; i < count; ++i) {
        seg.packed[i] = packed[i];
        seg.scales[i] = scales[i];
        seg.y[i] = y[i];
        seg.n[i] = n[i];
        seg.tiles_n[i] = (n[i] + BN - 1) / BN;
        seg.tile0[i] = tiles;
        tiles += seg.tiles_n[i] * ((m + BM - 1) / BM);
        sv = sv && (reinterpret_cast<uintptr_t>(scales[i]) % 4) == 0;
        if ((reinterpret_cast<uintptr_t>(y[i]) % 16) != 0 || n[i] % 4 != 0) vec = 0;
    }
    constexpr bool kSv = SvOk<MB, NB, WN, WK, KG, S>::value;
    if ((k / 32) % KG != 0)
        return launch_gemm32_grid<MB, NB, WN, WK, KG, S, false, true>(x, seg, tiles, m, k, vec,
                                                                      stream);
    if (sv) return launch_gemm32_grid<MB, NB, WN, WK, KG, S, kSv, false>(x, seg, tiles, m, k, vec,
                                                                          stream);
    return launch_gemm32_grid<MB, NB, WN, WK, KG, S, false, false>(x, seg, tiles, m, k, vec,
                                                                   stream);
}

// Tile shapes for m > 32, largest first, with the time one full round of
// them takes (k = 2560, n = 4096, one tile per CU, measured on MI355X: m =
// 1024, 512, 256 and 128 respectively).  All four are 32 x 32 block tiles; the
// two smaller ones replaced 16 x 16 block tiles of the same sizes (m = 256:
// 16.5 -> 12.4 us, m = 128: 12.5 -> 11.3 us).  The 32 x 64 tile splits K over
// eight waves (two per SIMD) with 16-group stages: its four-wave, 8-group,
// three-stage form waited on its loads (m = 48..128: 10.6-11.0 -> 8.5-9.0 us
// with cache-resident weights), and with the weights read from HBM a third
// stage in the ring pays (m = 128: 11.3 -> 10.7 us; 8-group stages in rings
// of 4 or 6: 12.1 / 13.1 us).
constexpr TileChoice kTiles[] = {
    {128, 128, 35.f},      // gemm32_kernel<4, 1, 4, 2, 4, 3>: 4 column slices x 2 K phases
    {64, 128, 19.f},       // gemm32_kernel<2, 2, 2, 4, 8, 2>: 2 column slices x 4 K phases
    {64, 64, 12.5f},       // gemm32_kernel<2, 1, 2, 4, 8, 3>: 2 column slices x 4 K phases
    {32, 64, 9.0f},        // gemm32_kernel<1, 2, 1, 8, 16, 3>: 1 column slice x 8 K phases
};

hipError_t launch_gemm_segments(const uint16_t* x, int count, const uint8_t* const* packed,
                                const uint16_t* const* scales, float* const* y,
                                const int64_t* n, int64_t m, int64_t k, hipStream_t stream) {
    if (m <= 16)      // 16 x 16 tiles: the weight traffic of a small batch spread over every CU
        return launch_gemm_small(x, count, packed, scales, y, n, m, k, stream);
    if (m <= 32)      // 32 x 16 tiles (measured 10.5 -> 8.0 us at m = 32, n = 4096, k = 2560)
        return launch_gemm_t<32, 1, 4, 4, 3, 1>(x, count, packed, scales, y, n, m, k, stream);
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    switch (choose_tile(kTiles, 4, m, count, n, device_info(dev).cu_count)) {
        case 0: return launch_gemm32_t<4, 1, 4, 2, 4, 3>(x, count, packed, scales, y, n, m, k, stream);
        case 1: return launch_gemm32_t<2, 2, 2, 4, 8, 2>(x, count, packed, scales, y, n, m, k, stream);
        case 2: return launch_gemm32_t<2, 1, 2, 4, 8, 3>(x, count, packed, scales, y, n, m, k, stream);
        default: return launch_gemm32_t<1, 2, 1, 8, 16, 3>(x, count, packed, scales, y, n, m, k, stream);
    }
}

}  // namespace

hipError_t launch_gemm_small(const uint16_t* x, int count, const uint8_t* const* packed,
                             const uint16_t* const* scales, float* const* y, const int64_t* n,
                             int64_t m, int64_t k, hipStream_t stream) {
    return launch_gemm_t<16, 1, 4, 4, 4, 1>(x, count, packed, scales, y, n, m, k, stream);
}

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
