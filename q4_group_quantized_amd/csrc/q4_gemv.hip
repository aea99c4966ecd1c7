// q4_gemv.hip -- decode-time Q4 product y[m, n] = sum_j s[n, j] * <x[m, group j], q[n, group j]>
// for 1 <= m <= 8 on gfx950.
//
// Method: the Q4 GEMV the QORA engines run for every projection and for the
// LM head (QORA-LLM-0.8B model card, "AVX-512 SIMD Acceleration", Q4 GEMV
// row: a 16-entry table lookup per 4-bit code; QORA-4B article, quantization
// section: symmetric 4-bit, group size 32).  The card's kernel is an AVX-512
// loop over rows; here the same arithmetic is laid out for CDNA4.
//
// Work split.  One wave owns a block of 16 weight rows and walks the whole K
// dimension in tiles of 8 groups (256 elements).  Lane l serves row
// n = 16*blk + (l % 16) and "slot" kb = l / 16; per tile it issues two 16-byte
// loads, the whole group (n, j0+kb) and the whole group (n, j0+4+kb), so every
// byte loaded is used and a wave load covers 16 rows x 64 contiguous bytes.
//
// Block-diagonal MFMA.  v_mfma_f32_16x16x32_f16 reduces over K = 32 split in
// four 8-wide slots, slot kb supplied by lanes 16*kb..16*kb+15.  Lane (n, kb)
// supplies, as B, eight codes of ITS OWN group (n, j0+kb) -- dword t of the
// group for the t-th of four chained MFMAs.  The A operand has 16 rows; row
// 4*tau + s holds token tau's activations of group j0+s in slot s and zeros in
// the other three slots.  After the four MFMAs, D[4*tau + s][n] is exactly the
// 32-term dot product of token tau with group (n, j0+s), kept apart from the
// other three groups, so each group's scale is applied in fp32 afterwards:
// acc += sum_s scale[n, j0+s] * D[4*tau+s][n].  In the D layout lane l holds
// rows 4*(l/16)+v, i.e. token l/16 and the four groups of its row: no
// cross-lane reduction is ever needed.  Tokens 4..7 use a second A operand and
// a second MFMA chain on the same unpacked B.
//
// Activations are staged once per workgroup in LDS, permuted inside every
// 8-element chunk to the order unpack8 produces codes in, so A and B agree
// element by element.  Scales are read as 8 consecutive fp16 per lane (one
// 16-byte load when the scale rows are 16-byte aligned).
//
// m = 1 has its own streaming kernel (gemv1_kernel below): there the block-
// diagonal MFMA would waste 15/16 of the matrix core anyway, and what bounds
// the kernel is how sequentially each wave walks HBM.  Every wave owns a
// contiguous range of rows and reads it front to back; LPR = 8, 16 or 32
// lanes share a row, each lane owning the same GPL = K / (32 LPR) groups of
// every row, so its activations stay in registers for the whole kernel.
// Per group: 16-byte code load, the 16-entry table lookup as four fp16 pairs,
// four v_dot2_f32_f16 against the matching activation pairs, then the fp32
// scale; the 16 per-lane partial sums of a row are added with DPP rotations.
#include "q4_device.hpp"
#include "q4_launch.hpp"

namespace q4 {
namespace {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kTileGroups = 8;                  // groups per tile (two sets of 4)
constexpr int kLdsBudget = 64 * 1024;           // bytes of LDS for activations
constexpr int kPrefetch = 4;                    // tiles in flight per wave

struct Tile {
    u32x4_t p0;      // group j0 + kb
    u32x4_t p1;      // group j0 + 4 + kb
    u32x4_t sc;      // fp16 scales of groups j0 .. j0+7 (row n)
};

// Loads of one tile, without branches so that a wave can keep several tiles
// in flight: `prow`/`srow` always point at a real row (callers clamp rows past
// N to row N-1 and never store those results) and groups past G are clamped to
// G-1 -- their activations in LDS are zero, so they add exactly nothing.
template <bool kScale16>
__device__ __forceinline__ Tile load_tile(const uint8_t* __restrict__ prow,
                                          const uint16_t* __restrict__ srow,
                                          int j0, int kb, int G) {
    Tile t;
    const int ja = min(j0 + kb, G - 1), jb = min(j0 + 4 + kb, G - 1);
    t.p0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(prow + 16 * ja));
    t.p1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(prow + 16 * jb));
    if (kScale16) {                              // G % 8 == 0: the tile is whole
        t.sc = *reinterpret_cast<const u32x4_t*>(srow + j0);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) h[v] = srow[min(j0 + v, G - 1)];
        t.sc = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                       h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
    return t;
}

// xs: LDS activations [TB*4 tokens][cg groups][32 halves, unpack order],
// followed by 32 zero halves that off-diagonal lanes read as their A operand.
template <int TB>
__device__ __forceinline__ void compute_tile(const Tile& t, const _Float16* xs,
                                             int cg, int jl0, int lane,
                                             half8_t (&a)[TB][4], float (&acc)[TB]) {
    const int kb = lane >> 4;
    const bool diag = (lane & 3) == kb;          // A row (lane%16) = 4*tau + slot
    const int tau_a = (lane & 15) >> 2;
    float s[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        s[2 * v] = half_bits_to_float(t.sc[v] & 0xFFFFu);
        s[2 * v + 1] = half_bits_to_float(t.sc[v] >> 16);
    }
#pragma unroll
    for (int set = 0; set < 2; ++set) {
        const u32x4_t p = set ? t.p1 : t.p0;
        half8_t b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = unpack8(p[q]);
        const int jl = jl0 + 4 * set + kb;       // local group of this lane's A slot
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const half8_t* src = reinterpret_cast<const half8_t*>(
                diag ? xs + ((size_t)(4 * tb + tau_a) * cg + jl) * 32
                     : xs + (size_t)TB * 4 * cg * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q) a[tb][q] = src[q];
            float4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tb][q], b[q], d, 0, 0, 0);
            float r = acc[tb];
#pragma unroll
            for (int v = 0; v < 4; ++v) r = fmaf(s[4 * set + v], d[v], r);
            acc[tb] = r;
        }
    }
}

// Stage activations of groups [jc0, jc0 + cg) of all TB*4 token slots into
// LDS, permuted to unpack order; tokens >= M and groups >= G are zero.
template <int TB>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, _Float16* xs, int M,
                                        int K, int G, int jc0, int cg) {
    const int units = TB * 4 * cg * 4;                  // 16-byte units
    for (int u = threadIdx.x; u < units; u += kGemvThreads) {
        const int q = u & 3;
        const int jl = (u >> 2) % cg;
        const int tok = (u >> 2) / cg;
        u32x4_t v = {0u, 0u, 0u, 0u};
        const int j = jc0 + jl;
        if (tok < M && j < G)
            v = *reinterpret_cast<const u32x4_t*>(x + (size_t)tok * K + 32 * j + 8 * q);
        *reinterpret_cast<u32x4_t*>(xs + ((size_t)tok * cg + jl) * 32 + 8 * q) = permute_x8(v);
    }
    if (threadIdx.x < 4)
        *reinterpret_cast<u32x4_t*>(xs + (size_t)TB * 4 * cg * 32 + 8 * threadIdx.x) =
            u32x4_t{0u, 0u, 0u, 0u};
}

template <int TB>
__device__ __forceinline__ void store_rows(float* __restrict__ y, const float (&acc)[TB],
                                           int64_t rb, int lane, int M, int64_t N) {
    const int64_t n = rb * 16 + (lane & 15);
    if (n < N) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int tok = 4 * tb + (lane >> 4);       // D row block = token
            if (tok < M) y[(int64_t)tok * N + n] = acc[tb];
        }
    }
}

// Whole K in one LDS pass.  Each wave owns a contiguous, balanced range of
// row blocks and streams it as one flat sequence of (row block, tile) steps;
// the prefetch ring runs across row-block boundaries, so a wave's loads never
// drain until its range is done.
template <int TB, bool kScale16>
__device__ __forceinline__ void gemv_flat(const uint16_t* __restrict__ x,
                                          const uint8_t* __restrict__ packed,
                                          const uint16_t* __restrict__ scales,
                                          float* __restrict__ y, _Float16* xs, int M,
                                          int64_t N, int K, int G, int64_t RB) {
    const int lane = threadIdx.x & 63;
    const int kb = lane >> 4;
    const int64_t W = (int64_t)gridDim.x * kGemvWaves;
    const int64_t w = (int64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6);
    const int64_t base = RB / W, extra = RB % W;
    const int64_t rb_begin = w * base + (w < extra ? w : extra);
    const int64_t count = base + (w < extra ? 1 : 0);
    const int T = ((G + 7) & ~7) / kTileGroups;          // tiles per row block
    const int64_t F = count * T;                         // flat steps of this wave

    // load cursor; steps past the wave's range re-read row N-1 (see load_tile)
    const int64_t rb_end = rb_begin + count;
    int64_t lrb = rb_begin;
    int lt = 0;
    auto load_next = [&]() -> Tile {
        const int64_t n = lrb * 16 + (lane & 15);
        const int64_t nc = (lrb < rb_end && n < N) ? n : N - 1;
        Tile t = load_tile<kScale16>(packed + nc * (int64_t)(K / 2), scales + nc * (int64_t)G,
                                     lt * kTileGroups, kb, G);
        if (++lt == T) { lt = 0; ++lrb; }
        return t;
    };

    Tile ring[kPrefetch];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) ring[p] = load_next();

    stage_x<TB>(x, xs, M, K, G, 0, T * kTileGroups);
    __syncthreads();

    half8_t a[TB][4];
    float acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = 0.f;
    int64_t crb = rb_begin;
    int ct = 0;
    const int cg = T * kTileGroups;
    for (int64_t f0 = 0; f0 < F; f0 += kPrefetch) {
#pragma unroll
        for (int p = 0; p < kPrefetch; ++p) {
            if (f0 + p < F)
                compute_tile<TB>(ring[p], xs, cg, ct * kTileGroups, lane, a, acc);
            ring[p] = load_next();
            if (f0 + p < F && ++ct == T) {
                store_rows<TB>(y, acc, crb, lane, M, N);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) acc[tb] = 0.f;
                ct = 0;
                ++crb;
            }
        }
    }
}

// K larger than one LDS pass: activations are staged chunk by chunk, with
// block-wide barriers, so every wave of a block walks the same number of
// row-block iterations.
template <int TB, bool kScale16>
__device__ __forceinline__ void gemv_chunked(const uint16_t* __restrict__ x,
                                             const uint8_t* __restrict__ packed,
                                             const uint16_t* __restrict__ scales,
                                             float* __restrict__ y, _Float16* xs, int M,
                                             int64_t N, int K, int G, int chunk_groups,
                                             int nchunks, int64_t RB) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kb = lane >> 4;
    const int64_t per_round = (int64_t)gridDim.x * kGemvWaves;
    const int64_t iters = (RB + per_round - 1) / per_round;
    half8_t a[TB][4];
    for (int64_t it = 0; it < iters; ++it) {
        const int64_t rb = (it * gridDim.x + blockIdx.x) * kGemvWaves + wave;
        const int64_t n = rb * 16 + (lane & 15);
        const int64_t nc = (rb < RB && n < N) ? n : N - 1;
        const uint8_t* prow = packed + nc * (int64_t)(K / 2);
        const uint16_t* srow = scales + nc * (int64_t)G;
        float acc[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb] = 0.f;
        for (int c = 0; c < nchunks; ++c) {
            const int jc0 = c * chunk_groups;
            const int cg = min(chunk_groups, ((G + 7) & ~7) - jc0);
            __syncthreads();
            stage_x<TB>(x, xs, M, K, G, jc0, cg);
            __syncthreads();
            if (rb < RB) {
                const int ntiles = cg / kTileGroups;
                Tile ring[kPrefetch];
#pragma unroll
                for (int p = 0; p < kPrefetch; ++p)
                    if (p < ntiles)
                        ring[p] = load_tile<kScale16>(prow, srow, jc0 + p * kTileGroups, kb, G);
                for (int t0 = 0; t0 < ntiles; t0 += kPrefetch) {
#pragma unroll
                    for (int p = 0; p < kPrefetch; ++p) {
                        const int tt = t0 + p;
                        if (tt < ntiles) {
                            compute_tile<TB>(ring[p], xs, cg, tt * kTileGroups, lane, a, acc);
                            if (tt + kPrefetch < ntiles)
                                ring[p] = load_tile<kScale16>(
                                    prow, srow, jc0 + (tt + kPrefetch) * kTileGroups, kb, G);
                        }
                    }
                }
            }
        }
        if (rb < RB) store_rows<TB>(y, acc, rb, lane, M, N);
    }
}

template <int TB, bool kScale16>
__global__ __launch_bounds__(kGemvThreads, 2) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int M, int64_t N, int K,
    int G, int chunk_groups, int nchunks, int64_t RB) {
    extern __shared__ __align__(16) unsigned char smem[];
    _Float16* xs = reinterpret_cast<_Float16*>(smem);
    if (nchunks == 1)
        gemv_flat<TB, kScale16>(x, packed, scales, y, xs, M, N, K, G, RB);
    else
        gemv_chunked<TB, kScale16>(x, packed, scales, y, xs, M, N, K, G, chunk_groups, nchunks,
                                   RB);
}

template <int TB, bool kScale16>
hipError_t launch_gemv_t(const uint16_t* x, const uint8_t* packed,
                         const uint16_t* scales, float* y, int m, int64_t n,
                         int k, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int G = k / 32;
    const int gpad = (G + 7) & ~7;
    const int per_group_bytes = TB * 4 * 64;
    int chunk = (kLdsBudget / per_group_bytes) & ~7;
    if (chunk > gpad) chunk = gpad;
    const int nchunks = (gpad + chunk - 1) / chunk;
    const int64_t RB = (n + 15) / 16;
    // resident waves: 4 per SIMD, 4 SIMDs per CU
    const int64_t max_waves = (int64_t)device_info(dev).cu_count * 16;
    int64_t waves;
    if (nchunks == 1) {
        // as many waves as fit, then trimmed so that every wave gets the same
        // number of row blocks (ceil(RB / waves) blocks each)
        const int64_t per = (RB + max_waves - 1) / max_waves;
        waves = (RB + per - 1) / per;
    } else {
        waves = RB < max_waves ? RB : max_waves;
    }
    const int64_t blocks64 = (waves + kGemvWaves - 1) / kGemvWaves;
    const int blocks = (int)(blocks64 > 0 ? blocks64 : 1);
    const size_t lds = (size_t)per_group_bytes * chunk + 64;
    hipLaunchKernelGGL((gemv_kernel<TB, kScale16>), dim3(blocks), dim3(kGemvThreads), lds,
                       stream, x, packed, scales, y, m, n, k, G, chunk, nchunks, RB);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// m = 1 streaming kernel
// ---------------------------------------------------------------------------

constexpr int kGemv1MaxGpl = 8;                 // groups per lane

// Sum over aligned groups of LPR lanes (8, 16 or 32); every lane of the group
// receives the total.
template <int LPR>
__device__ __forceinline__ float lanes_sum(float v) {
    if (LPR == 8) {
        // xor 1 and xor 2 inside quads, then the mirror inside 8-lane halves
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
        return v;
    } else if (LPR == 16) {
        return row16_sum(v);
    } else {
        v = row16_sum(v);
        return v + __shfl_xor(v, 16, 64);
    }
}

// LPR lanes share a row (64 / LPR rows per wave step); lane `sub` owns groups
// sub + LPR * i, i < GPL, of every row, so G = LPR * GPL.  PF steps in flight.
template <int LPR, int GPL, int PF>
__global__ __launch_bounds__(kGemvThreads) void gemv1_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int64_t N, int K,
    int64_t RQ, SpliceConsts kc) {
    constexpr int RPS = 64 / LPR;                       // rows per wave step
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;
    const int r = lane / LPR;
    const int G = K / 32;
    const int64_t W = (int64_t)gridDim.x * kGemvWaves;
    const int64_t w = (int64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6);
    const int64_t base = RQ / W, extra = RQ % W;
    const int64_t q0 = w * base + (w < extra ? w : extra);
    const int64_t cnt = base + (w < extra ? 1 : 0);

    // this lane's activations, as fp16 pairs in unpack order
    uint32_t xr[GPL][16];
#pragma unroll
    for (int i = 0; i < GPL; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4_t v = permute_x8(*reinterpret_cast<const u32x4_t*>(
                x + 32 * (sub + LPR * i) + 8 * c));
#pragma unroll
            for (int e = 0; e < 4; ++e) xr[i][4 * c + e] = v[e];
        }

    // Loads stay unconditional so that PF steps remain in flight: steps past
    // the wave's range, and rows past N, re-read row N-1, which every wave
    // shares and the caches keep; those results are never stored.
    const int64_t row0 = RPS * q0 + r;
    const uint8_t* pbase = packed + row0 * (int64_t)(K / 2) + 16 * sub;
    const uint16_t* sbase = scales + row0 * (int64_t)G + sub;
    const uint8_t* plast = packed + (N - 1) * (int64_t)(K / 2) + 16 * sub;
    const uint16_t* slast = scales + (N - 1) * (int64_t)G + sub;
    const int64_t pstep = (int64_t)RPS * (K / 2);
    const int64_t sstep = (int64_t)RPS * G;
    u32x4_t rp[PF][GPL];
    uint32_t rs[PF][GPL];
    auto load = [&](int slot, int64_t f) {
        const bool ok = f < cnt && row0 + RPS * f < N;
        const uint8_t* pp = ok ? pbase + f * pstep : plast;
        const uint16_t* sp = ok ? sbase + f * sstep : slast;
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            rp[slot][i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(pp + 16 * LPR * i));
            rs[slot][i] = sp[LPR * i];
        }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, p);

    const uint32_t mask = kc.mask;
    const uint32_t magic = to_vgpr(kc.magic);
    for (int64_t f0 = 0; f0 < cnt; f0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int64_t f = f0 + p;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                float dot = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    half2_t h[4];
                    unpack8_pairs(rp[p][i][c], mask, magic, h);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dot = __builtin_amdgcn_fdot2(h[e], as_half2(xr[i][4 * c + e]), dot,
                                                     false);
                }
                acc = fmaf(half_bits_to_float(rs[p][i]), dot, acc);
            }
            load(p, f + PF);
            acc = lanes_sum<LPR>(acc);
            const int64_t row = row0 + RPS * f;
            if (f < cnt && sub == 0 && row < N) y[row] = acc;
        }
    }
}

template <int LPR, int GPL>
hipError_t launch_gemv1_t(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                          float* y, int64_t n, int k, hipStream_t stream) {
    constexpr int PF = GPL <= 4 ? 4 : 2;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    constexpr int RPS = 64 / LPR;
    const int64_t RQ = (n + RPS - 1) / RPS;
    static int blocks_per_cu = 0;               // occupancy of this instantiation
    if (blocks_per_cu == 0) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, gemv1_kernel<LPR, GPL, PF>,
                                                         kGemvThreads, 0) != hipSuccess ||
            nb < 1)
            nb = 1;
        blocks_per_cu = nb;
    }
    // as many waves as are resident at once, trimmed so that every wave gets
    // the same number of steps
    const int64_t max_waves = (int64_t)device_info(dev).cu_count * blocks_per_cu * kGemvWaves;
    const int64_t per = (RQ + max_waves - 1) / max_waves;
    const int64_t waves = (RQ + per - 1) / per;
    const int blocks = (int)((waves + kGemvWaves - 1) / kGemvWaves);
    hipLaunchKernelGGL((gemv1_kernel<LPR, GPL, PF>), dim3(blocks), dim3(kGemvThreads), 0, stream,
                       x, packed, scales, y, n, k, RQ, kSpliceConsts);
    return hipGetLastError();
}

template <int LPR>
hipError_t launch_gemv1_lpr(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                            float* y, int64_t n, int k, hipStream_t stream) {
    switch ((k / 32) / LPR) {
        case 1: return launch_gemv1_t<LPR, 1>(x, packed, scales, y, n, k, stream);
        case 2: return launch_gemv1_t<LPR, 2>(x, packed, scales, y, n, k, stream);
        case 3: return launch_gemv1_t<LPR, 3>(x, packed, scales, y, n, k, stream);
        case 4: return launch_gemv1_t<LPR, 4>(x, packed, scales, y, n, k, stream);
        case 5: return launch_gemv1_t<LPR, 5>(x, packed, scales, y, n, k, stream);
        case 6: return launch_gemv1_t<LPR, 6>(x, packed, scales, y, n, k, stream);
        case 7: return launch_gemv1_t<LPR, 7>(x, packed, scales, y, n, k, stream);
        default: return launch_gemv1_t<LPR, 8>(x, packed, scales, y, n, k, stream);
    }
}

// Lanes per row for the m = 1 kernel, or 0 when k does not fit it.  Short
// rows (k <= 1024) use 8 lanes per row so that each lane still owns 4 groups.
int gemv1_lanes_per_row(int64_t k) {
    const int64_t G = k / 32;
    if (G % 8 == 0 && G <= 32) return 8;
    if (G % 16 == 0 && G / 16 <= kGemv1MaxGpl) return 16;
    if (G % 8 == 0 && G / 8 <= kGemv1MaxGpl) return 8;
    if (G % 32 == 0 && G / 32 <= kGemv1MaxGpl) return 32;
    return 0;
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed,
                       const uint16_t* scales, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
    const int64_t G = k / 32;
    if (m == 1) {
        switch (gemv1_lanes_per_row(k)) {
            case 8: return launch_gemv1_lpr<8>(x, packed, scales, y, n, (int)k, stream);
            case 16: return launch_gemv1_lpr<16>(x, packed, scales, y, n, (int)k, stream);
            case 32: return launch_gemv1_lpr<32>(x, packed, scales, y, n, (int)k, stream);
            default: break;
        }
    }
    const bool s16 = (G % 8) == 0;
    if (m <= 4)
        return s16 ? launch_gemv_t<1, true>(x, packed, scales, y, (int)m, n, (int)k, stream)
                   : launch_gemv_t<1, false>(x, packed, scales, y, (int)m, n, (int)k, stream);
    return s16 ? launch_gemv_t<2, true>(x, packed, scales, y, (int)m, n, (int)k, stream)
               : launch_gemv_t<2, false>(x, packed, scales, y, (int)m, n, (int)k, stream);
}

}  // namespace q4
