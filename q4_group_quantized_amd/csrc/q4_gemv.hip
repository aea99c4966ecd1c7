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

template <bool kScale16>
__device__ __forceinline__ Tile load_tile(const uint8_t* __restrict__ prow,
                                          const uint16_t* __restrict__ srow,
                                          int j0, int kb, int G, bool row_ok) {
    Tile t;
    const u32x4_t zero_codes = {0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u};
    t.p0 = zero_codes;
    t.p1 = zero_codes;
    t.sc = u32x4_t{0u, 0u, 0u, 0u};
    if (row_ok) {
        const int ja = j0 + kb, jb = j0 + 4 + kb;
        if (ja < G)
            t.p0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(prow + 16 * ja));
        if (jb < G)
            t.p1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(prow + 16 * jb));
        if (kScale16) {
            if (j0 + kTileGroups <= G) {
                t.sc = *reinterpret_cast<const u32x4_t*>(srow + j0);
            } else {
                uint32_t h[8];
#pragma unroll
                for (int v = 0; v < 8; ++v) h[v] = (j0 + v < G) ? srow[j0 + v] : 0u;
                t.sc = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                               h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
            }
        } else {
            uint32_t h[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) h[v] = (j0 + v < G) ? srow[j0 + v] : 0u;
            t.sc = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                           h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
    }
    return t;
}

// xs: LDS activations [TB*4 tokens][cg groups][32 halves, unpack order]
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
            if (diag) {
                const half8_t* src = reinterpret_cast<const half8_t*>(
                    xs + ((size_t)(4 * tb + tau_a) * cg + jl) * 32);
#pragma unroll
                for (int q = 0; q < 4; ++q) a[tb][q] = src[q];
            }
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

template <int TB, bool kScale16>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int M,
    int64_t N, int K, int G, int chunk_groups, int nchunks, int64_t RB,
    int iters) {
    extern __shared__ __align__(16) unsigned char smem[];
    _Float16* xs = reinterpret_cast<_Float16*>(smem);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kb = lane >> 4;

    half8_t a[TB][4];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int q = 0; q < 4; ++q) a[tb][q] = half8_t{0, 0, 0, 0, 0, 0, 0, 0};

    for (int it = 0; it < iters; ++it) {
        const int64_t rb = ((int64_t)it * gridDim.x + blockIdx.x) * kGemvWaves + wave;
        const int64_t n = rb * 16 + (lane & 15);
        const bool row_ok = (rb < RB) && (n < N);
        const uint8_t* prow = packed + (row_ok ? n : 0) * (int64_t)(K / 2);
        const uint16_t* srow = scales + (row_ok ? n : 0) * (int64_t)G;
        float acc[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb] = 0.f;

        for (int c = 0; c < nchunks; ++c) {
            const int jc0 = c * chunk_groups;
            const int cg = min(chunk_groups, ((G + 7) & ~7) - jc0);
            if (nchunks > 1 || it == 0) {
                if (it > 0 || c > 0) __syncthreads();
                // stage activations of groups [jc0, jc0+cg) for TB*4 tokens
                const int units = TB * 4 * cg * 4;          // 16-byte units
                for (int u = threadIdx.x; u < units; u += kGemvThreads) {
                    const int q = u & 3;
                    const int jl = (u >> 2) % cg;
                    const int tok = (u >> 2) / cg;
                    u32x4_t v = {0u, 0u, 0u, 0u};
                    const int j = jc0 + jl;
                    if (tok < M && j < G)
                        v = *reinterpret_cast<const u32x4_t*>(x + (size_t)tok * K + 32 * j + 8 * q);
                    *reinterpret_cast<u32x4_t*>(xs + ((size_t)tok * cg + jl) * 32 + 8 * q) =
                        permute_x8(v);
                }
                __syncthreads();
            }
            if (rb < RB) {
                const int ntiles = cg / kTileGroups;
                Tile ring[kPrefetch];
#pragma unroll
                for (int p = 0; p < kPrefetch; ++p)
                    if (p < ntiles)
                        ring[p] = load_tile<kScale16>(prow, srow, jc0 + p * kTileGroups, kb, G, row_ok);
                for (int t0 = 0; t0 < ntiles; t0 += kPrefetch) {
#pragma unroll
                    for (int p = 0; p < kPrefetch; ++p) {
                        const int tt = t0 + p;
                        if (tt < ntiles) {
                            compute_tile<TB>(ring[p], xs, cg, tt * kTileGroups, lane, a, acc);
                            if (tt + kPrefetch < ntiles)
                                ring[p] = load_tile<kScale16>(prow, srow,
                                                              jc0 + (tt + kPrefetch) * kTileGroups,
                                                              kb, G, row_ok);
                        }
                    }
                }
            }
        }
        if (row_ok) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int tok = 4 * tb + kb;            // D row block = token
                if (tok < M) y[(int64_t)tok * N + n] = acc[tb];
            }
        }
    }
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
    const int64_t want = (RB + kGemvWaves - 1) / kGemvWaves;
    const int64_t cap = (int64_t)device_info(dev).cu_count * 4;
    const int blocks = (int)(want < cap ? want : cap);
    const int iters = (int)((RB + (int64_t)blocks * kGemvWaves - 1) / ((int64_t)blocks * kGemvWaves));
    const size_t lds = (size_t)per_group_bytes * chunk;
    hipLaunchKernelGGL((gemv_kernel<TB, kScale16>), dim3(blocks), dim3(kGemvThreads), lds,
                       stream, x, packed, scales, y, m, n, k, G, chunk, nchunks, RB, iters);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed,
                       const uint16_t* scales, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
    const bool s16 = ((k / 32) % 8) == 0;
    if (m <= 4)
        return s16 ? launch_gemv_t<1, true>(x, packed, scales, y, (int)m, n, (int)k, stream)
                   : launch_gemv_t<1, false>(x, packed, scales, y, (int)m, n, (int)k, stream);
    return s16 ? launch_gemv_t<2, true>(x, packed, scales, y, (int)m, n, (int)k, stream)
               : launch_gemv_t<2, false>(x, packed, scales, y, (int)m, n, (int)k, stream);
}

}  // namespace q4
