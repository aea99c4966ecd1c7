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
// 8-element chunk to the order unpack8_fma produces codes in, so A and B agree
// element by element; several matrices over the same x (q4_gemv_multi) share
// one launch, their waves split in proportion to their rows.  Scales are read as 8 consecutive fp16 per lane (one
// 16-byte load when G % 8 == 0 and the scale matrix is 16-byte aligned, else
// eight 2-byte loads).
//
// At m = 2..8 a matrix of at most kGemvTileRows rows is handed to the GEMM's
// small-batch kernel instead (launch_gemm_small): with one 16-row block per
// wave walking all of K, a few thousand rows would leave most of the
// device idle.
//
// m = 1 has its own streaming kernel (gemv1_kernel below): there the block-
// diagonal MFMA would waste 15/16 of the matrix core anyway, and what bounds
// the kernel is how sequentially each wave walks HBM.  Every wave owns a
// contiguous range of rows and reads it front to back, one or two waves per
// SIMD (see gemv1_waves_per_simd); LPR = 16, 8 or 32 lanes share a row, each lane owning the same
// GPL = K / (32 LPR) groups of every row, so its activations stay in
// registers for the whole kernel.  Per group: 16-byte code load, the 16-entry
// table lookup as fp16 pairs (unpack8_split), v_dot2_f32_f16 against the
// matching activation pairs into two fp32 sums, then the fp32 scale; the
// per-lane partial sums of a row are added with DPP rotations.  The same
// kernel serves several matrices that share x (q4_gemv_multi) from a table
// of segments, so a set of projections costs one launch.
#include "q4.h"
#include "q4_device.hpp"
#include "q4_launch.hpp"
#include "q4_topk.hpp"

namespace q4 {
namespace {

constexpr int kGemvWaves = 4;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kTileGroups = 8;                  // groups per tile (two sets of 4)
constexpr int kLdsBudget = 64 * 1024;           // bytes of LDS for activations
constexpr int kPrefetch = 4;                    // tiles in flight per wave
// Halves of padding after each token's activations in LDS: with rows of
// 64-byte groups the token stride would be a multiple of the 256-byte bank
// span, so the four tokens read by one MFMA operand would hit the same banks.
constexpr int kTokenPad = 8;

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
    if (kScale16) {                              // G % 8 == 0 and 16-byte aligned scales
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

// xs: LDS activations [TB*4 tokens][cg groups][32 halves, unpack order], each
// token's row followed by kTokenPad halves, then 32 zero halves that
// off-diagonal lanes read as their A operand.
template <int TB>
__device__ __forceinline__ void compute_tile(const Tile& t, const _Float16* xs,
                                             int cg, int jl0, int lane, uint32_t mask,
                                             uint32_t mask16, uint32_t magic,
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
        for (int q = 0; q < 4; ++q) b[q] = unpack8_fma(p[q], mask, mask16, magic);
        const int jl = jl0 + 4 * set + kb;       // local group of this lane's A slot
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const half8_t* src = reinterpret_cast<const half8_t*>(
                diag ? xs + (size_t)(4 * tb + tau_a) * (cg * 32 + kTokenPad) + jl * 32
                     : xs + (size_t)TB * 4 * (cg * 32 + kTokenPad));
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
// Loads are issued kStageBatch at a time before any of them is written, so a
// thread waits for one round trip per batch rather than one per 16 bytes
// (at k = 2560 and m = 8 a thread moves ten units; staged one by one they
// cost several microseconds before the first product).
constexpr int kStageBatch = 8;

template <int TB>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, _Float16* xs, int M,
                                        int K, int G, int jc0, int cg) {
    const int units = TB * 4 * cg * 4;                  // 16-byte units
    for (int u0 = threadIdx.x; u0 < units; u0 += kStageBatch * kGemvThreads) {
        u32x4_t v[kStageBatch];
        int off[kStageBatch];
#pragma unroll
        for (int b = 0; b < kStageBatch; ++b) {
            const int u = u0 + b * kGemvThreads;
            const int q = u & 3;
            const int jl = (u >> 2) % cg;
            const int tok = (u >> 2) / cg;
            const int j = jc0 + jl;
            v[b] = u32x4_t{0u, 0u, 0u, 0u};
            if (u < units && tok < M && j < G)
                v[b] = *reinterpret_cast<const u32x4_t*>(x + (size_t)tok * K + 32 * j + 8 * q);
            off[b] = u < units ? tok * (cg * 32 + kTokenPad) + jl * 32 + 8 * q : -1;
        }
#pragma unroll
        for (int b = 0; b < kStageBatch; ++b)
            if (off[b] >= 0) *reinterpret_cast<u32x4_t*>(xs + off[b]) = permute_x8(v[b]);
    }
    if (threadIdx.x < 4)
        *reinterpret_cast<u32x4_t*>(xs + (size_t)TB * 4 * (cg * 32 + kTokenPad) + 8 * threadIdx.x) =
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
// row blocks and streams it as one flat sequence of (row block, step) steps;
// the prefetch ring runs across row-block boundaries, so a wave's loads never
// drain until its range is done.  A step is 16 rows x 16 groups (two tiles).
// The codes are read in whole 256-byte row segments -- lane (lr, lj) =
// (lane / 16, lane % 16) loads group 16 t + lj of row 4 i + lr, i < 4, so one
// wave load covers 4 rows x 256 contiguous bytes, where a load in the tile
// layout itself would cover 16 rows x 64 bytes (~5.3 TB/s for that pattern
// alone) -- and each step passes through a wave-private LDS tile into the
// per-lane tile layout: group j of row n at 256 n + 16 ((j + n) mod 16), a
// rotation that keeps the row-wise writes and the tile reads (lane (n, kb)
// reads groups 8 h + kb and 8 h + 4 + kb of row n) free of bank conflicts.
// Lane (lane / 4, lane % 4) loads four of its row's 16 scales of the step;
// the tile's eight scales of row n are read back as one 16-byte piece.  Two
// step buffers per wave alternate.  The arithmetic (compute_tile) and the
// order of every sum are those of the tile layout, so the results do not
// depend on the load path.
constexpr int kStepGroups = 16;
constexpr int kStepCodeBytes = 16 * 256;
constexpr int kStepBytes = kStepCodeBytes + 16 * 32;      // codes + scales of a step

// The matrices of one flat launch (q4_gemv: one; q4_gemv_multi: up to
// kFlatMaxSegments sharing x and K).  Matrix s owns the waves
// [w0[s], w0[s] + wn[s]) of the grid, which split its row blocks evenly.
constexpr int kFlatMaxSegments = 8;
struct FlatSegments {
    const uint8_t* packed[kFlatMaxSegments];
    const uint16_t* scales[kFlatMaxSegments];
    float* y[kFlatMaxSegments];
    int32_t n[kFlatMaxSegments];                 // rows (< 2^31)
    int32_t w0[kFlatMaxSegments];                // first wave
    int32_t wn[kFlatMaxSegments];                // waves
    int count;
};
static_assert(kFlatMaxSegments == Q4_MULTI_MAX, "segment table must hold Q4_MULTI_MAX matrices");

template <int TB, bool kWhole16>
__device__ __forceinline__ void gemv_flat(const uint16_t* __restrict__ x,
                                          const FlatSegments& seg, _Float16* xs,
                                          unsigned char* step_bufs, int M, int K, int G,
                                          const SpliceConsts& kc) {
    const int lane = threadIdx.x & 63;
    const int kb = lane >> 4, rr = lane & 15;             // tile layout
    const int lr = lane >> 4, lj = lane & 15;             // code loads
    const int sr = lane >> 2, sp = lane & 3;              // scale loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = (int)blockIdx.x * kGemvWaves + wave;
    // this wave's matrix (wave-uniform selects over constant indices)
    const uint8_t* __restrict__ packed = seg.packed[0];
    const uint16_t* __restrict__ scales = seg.scales[0];
    float* __restrict__ y = seg.y[0];
    int N = seg.n[0], w0 = seg.w0[0], W = seg.wn[0];
#pragma unroll
    for (int i = 1; i < kFlatMaxSegments; ++i)
        if (i < seg.count && w >= seg.w0[i]) {
            packed = seg.packed[i]; scales = seg.scales[i]; y = seg.y[i];
            N = seg.n[i]; w0 = seg.w0[i]; W = seg.wn[i];
        }
    const int64_t RB = ((int64_t)N + 15) / 16;
    const int64_t lw = w - w0;                           // >= W: a spare wave, no rows
    const int64_t base = RB / W, extra = RB % W;
    const int64_t rb_begin = lw < W ? lw * base + (lw < extra ? lw : extra) : RB;
    const int64_t count = lw < W ? base + (lw < extra ? 1 : 0) : 0;
    const int T = ((G + 15) & ~15) / kStepGroups;        // steps per row block
    const int64_t F = count * T;                         // flat steps of this wave
    unsigned char* bufs = step_bufs + (size_t)wave * 2 * kStepBytes;

    struct Step {
        u32x4_t v[4];                                    // codes, row 4 i + lr, group lj
        uint32_t s0, s1;                                 // scales 4 sp .. 4 sp + 3 of row sr
    };
    // load cursor, advanced with selects rather than branches: with a
    // branch-free loop body the compiler keeps the later steps' loads in
    // flight instead of waiting for every load at each step.  Steps past the
    // wave's range re-read row N-1; groups past G re-read group G-1 (their
    // activations in LDS are zero).
    //
    // Addressing: buffer loads from the row block's first row.  The block's
    // base and byte count are wave-uniform (scalar registers, rebuilt per
    // step); a lane adds a fixed 32-bit offset inside the block (row < 16,
    // K/2 <= 2^23 bytes per row).  Rows past N in the matrix's last block lie
    // past the buffer's end and read as zeros (their results are never
    // stored), so no lane clamps a row.  Steps past the wave's range re-read
    // its last row block.
    const int64_t rb_end = rb_begin + count;
    const int64_t rb_last = (rb_end > 0 ? rb_end : 1) - 1;
    int64_t lrb = rb_begin;
    int lt = 0;
    const int code_lane = lr * (K / 2) + 16 * lj;                // row lr, group lj of a step
    const int scale_lane = 2 * (sr * G + 4 * sp);                // row sr, groups 4 sp .. +3
    auto load_next = [&]() -> Step {
        Step st;
        const int64_t lb = lrb < rb_end ? lrb : rb_last;             // uniform
        const int64_t left = N - lb * 16;                            // rows from lb on, >= 1
        const int rows = (int)(left < 16 ? left : 16);
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(packed + lb * 16 * (int64_t)(K / 2)), (short)0, rows * (K / 2), kBufferFlags);
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(scales + lb * 16 * (int64_t)G), (short)0, rows * G * 2, kBufferFlags);
        // groups past G (last step, G % 16 != 0) re-read group G - 1 of the row
        const int g = lt * kStepGroups + lj;
        const int voff = kWhole16 ? code_lane : lr * (K / 2) + 16 * (g < G ? g : G - 1);
        const int soff = kWhole16 ? 16 * kStepGroups * lt : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            st.v[i] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                             crs, voff, soff + 4 * i * (K / 2), kBufferNontemporal));
        const int gs = lt * kStepGroups + 4 * sp;
        if (kWhole16) {                   // G % 16 == 0 (whole step), 8-byte aligned scales
            const uint2 v = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(srs, scale_lane,
                                                            2 * kStepGroups * lt, 0));
            st.s0 = v.x;
            st.s1 = v.y;
        } else {
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                h[e] = __builtin_amdgcn_raw_buffer_load_b16(
                    srs, 2 * (sr * G + (gs + e < G ? gs + e : G - 1)), 0, 0);
            st.s0 = h[0] | (h[1] << 16);
            st.s1 = h[2] | (h[3] << 16);
        }
        const int nt = lt + 1;
        const bool wrap = nt == T;
        lt = wrap ? 0 : nt;
        lrb += wrap ? 1 : 0;
        return st;
    };

    Step ring[kPrefetch];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) ring[p] = load_next();

    stage_x<TB>(x, xs, M, K, G, 0, T * kStepGroups);
    __syncthreads();

    const uint32_t magic = to_vgpr(kc.magic);
    half8_t a[TB][4];
    float acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = 0.f;
    int64_t crb = rb_begin;
    int ct = 0, sel = 0;
    const int cg = T * kStepGroups;
    // one step: through the wave's LDS buffer (the wave's own LDS accesses
    // are performed in order), then the two tiles; a finished row block is
    // stored
    auto compute_step = [&](const Step& st) {
        unsigned char* buf = bufs + sel * kStepBytes;
        sel ^= 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = 4 * i + lr;
            *reinterpret_cast<u32x4_t*>(buf + 256 * n + 16 * ((lj + n) & 15)) = st.v[i];
        }
        *reinterpret_cast<uint2*>(buf + kStepCodeBytes + 32 * sr + 8 * sp) = uint2{st.s0, st.s1};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            Tile t;
            t.p0 = *reinterpret_cast<const u32x4_t*>(buf + 256 * rr +
                                                     16 * ((8 * h + kb + rr) & 15));
            t.p1 = *reinterpret_cast<const u32x4_t*>(buf + 256 * rr +
                                                     16 * ((8 * h + 4 + kb + rr) & 15));
            t.sc = *reinterpret_cast<const u32x4_t*>(buf + kStepCodeBytes + 32 * rr + 16 * h);
            compute_tile<TB>(t, xs, cg, ct * kStepGroups + 8 * h, lane, kc.mask, kc.mask16,
                             magic, a, acc);
        }
        if (++ct == T) {
            store_rows<TB>(y, acc, crb, lane, M, N);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[tb] = 0.f;
            ct = 0;
            ++crb;
        }
    };
    // full rounds of kPrefetch steps, then the last steps with no new loads
    int64_t f0 = 0;
    for (; f0 + kPrefetch < F; f0 += kPrefetch) {
#pragma unroll
        for (int p = 0; p < kPrefetch; ++p) {
            compute_step(ring[p]);
            ring[p] = load_next();
        }
    }
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p)
        if (f0 + p < F) compute_step(ring[p]);
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
                                             int nchunks, int64_t RB, const SpliceConsts& kc) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kb = lane >> 4;
    const uint32_t magic = to_vgpr(kc.magic);
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
                            compute_tile<TB>(ring[p], xs, cg, tt * kTileGroups, lane, kc.mask,
                                             kc.mask16, magic, a, acc);
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

template <int TB, bool kWhole16>
__global__ __launch_bounds__(kGemvThreads, 2) void gemv_flat_kernel(
    const uint16_t* __restrict__ x, FlatSegments seg, int M, int K, int G, int xs_bytes,
    SpliceConsts kc) {
    extern __shared__ __align__(16) unsigned char smem[];
    gemv_flat<TB, kWhole16>(x, seg, reinterpret_cast<_Float16*>(smem), smem + xs_bytes, M, K,
                            G, kc);
}

template <int TB, bool kScale16>
__global__ __launch_bounds__(kGemvThreads, 2) void gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scales, float* __restrict__ y, int M, int64_t N, int K,
    int G, int chunk_groups, int nchunks, int64_t RB, SpliceConsts kc) {
    extern __shared__ __align__(16) unsigned char smem[];
    gemv_chunked<TB, kScale16>(x, packed, scales, y, reinterpret_cast<_Float16*>(smem), M, N, K,
                               G, chunk_groups, nchunks, RB, kc);
}

// Whole K staged at once when the padded activations and 2 step buffers per
// wave fit the CU's 160 KB of LDS (k <= 7680 at m = 5..8, 15360 at m <= 4):
// two workgroups per CU where their LDS allows (measured faster than one at
// k = 1024 and 2560), the waves split between the matrices in proportion to
// their row blocks, each wave of a matrix with the same number of row blocks.
// Otherwise chunked (kLdsBudget of activations per pass), as many waves as
// fit, one launch per matrix.
template <int TB>
hipError_t launch_gemv_t(const uint16_t* x, int m, int k, int count,
                         const uint8_t* const* packed, const uint16_t* const* scales,
                         float* const* y, const int64_t* n, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int cu = device_info(dev).cu_count;
    const int G = k / 32;
    const int per_group_bytes = TB * 4 * 64;
    const int fixed_bytes = TB * 4 * kTokenPad * 2 + 64;     // token pads, zero block
    const int64_t g16 = (G + 15) & ~15;
    const int64_t xs_bytes = (per_group_bytes * g16 + fixed_bytes + 15) & ~15;
    const size_t lds = (size_t)xs_bytes + (size_t)kGemvWaves * 2 * kStepBytes;
    if (lds <= (size_t)160 * 1024) {
        const int wgs = 2 * lds <= (size_t)160 * 1024 ? 2 : 1;
        const int64_t max_waves = (int64_t)cu * kGemvWaves * wgs;
        int64_t rb_total = 0;
        for (int s = 0; s < count; ++s) rb_total += (n[s] + 15) / 16;
        FlatSegments seg = {};
        seg.count = count;
        // 8-byte scale loads need whole steps and 8-byte aligned scale
        // matrices (the contract only promises 2 bytes)
        bool whole = G % 16 == 0;
        int64_t waves = 0;
        for (int s = 0; s < count; ++s) {
            const int64_t rb = (n[s] + 15) / 16;
            // this matrix's share of the resident waves, then as few waves
            // as give every wave the same number of row blocks
            int64_t share = (max_waves * rb + rb_total / 2) / rb_total;
            share = share < 1 ? 1 : share;
            const int64_t per = (rb + share - 1) / share;
            seg.packed[s] = packed[s];
            seg.scales[s] = scales[s];
            seg.y[s] = y[s];
            seg.n[s] = (int32_t)n[s];                    // n < 2^31 (checked by the API)
            seg.w0[s] = (int32_t)waves;
            seg.wn[s] = (int32_t)((rb + per - 1) / per);
            waves += seg.wn[s];
            whole = whole && (reinterpret_cast<uintptr_t>(scales[s]) & 7) == 0;
        }
        if (count == 1) {
            // one matrix: every wave of the grid takes a share
            seg.wn[0] = (int32_t)((waves + kGemvWaves - 1) / kGemvWaves * kGemvWaves);
        }
        const int blocks = (int)((waves + kGemvWaves - 1) / kGemvWaves);
        const void* fn = whole ? reinterpret_cast<const void*>(&gemv_flat_kernel<TB, true>)
                               : reinterpret_cast<const void*>(&gemv_flat_kernel<TB, false>);
        static std::atomic<uint64_t> lds_done[2] = {{0}, {0}};
        e = allow_dynamic_lds(fn, (int)lds, lds_done[whole ? 1 : 0]);
        if (e != hipSuccess) return e;
        if (whole)
            hipLaunchKernelGGL((gemv_flat_kernel<TB, true>), dim3(blocks), dim3(kGemvThreads), lds,
                               stream, x, seg, m, k, G, (int)xs_bytes, kSpliceConsts);
        else
            hipLaunchKernelGGL((gemv_flat_kernel<TB, false>), dim3(blocks), dim3(kGemvThreads),
                               lds, stream, x, seg, m, k, G, (int)xs_bytes, kSpliceConsts);
        return hipGetLastError();
    }
    const int gpad = (G + 7) & ~7;
    int chunk = ((kLdsBudget - fixed_bytes) / per_group_bytes) & ~7;
    if (chunk > gpad) chunk = gpad;
    const int nchunks = (gpad + chunk - 1) / chunk;
    const size_t chunk_lds = (size_t)per_group_bytes * chunk + fixed_bytes;
    for (int s = 0; s < count; ++s) {
        const int64_t RB = (n[s] + 15) / 16;
        // resident waves: 4 per SIMD, 4 SIMDs per CU
        const int64_t max_waves = (int64_t)cu * 16;
        const int64_t waves = RB < max_waves ? RB : max_waves;
        const int64_t blocks64 = (waves + kGemvWaves - 1) / kGemvWaves;
        const int blocks = (int)(blocks64 > 0 ? blocks64 : 1);
        if (G % 8 == 0 && (reinterpret_cast<uintptr_t>(scales[s]) & 15) == 0)   // 16-byte scale loads
            hipLaunchKernelGGL((gemv_kernel<TB, true>), dim3(blocks), dim3(kGemvThreads),
                               chunk_lds, stream, x, packed[s], scales[s], y[s], m, n[s], k, G,
                               chunk, nchunks, RB, kSpliceConsts);
        else
            hipLaunchKernelGGL((gemv_kernel<TB, false>), dim3(blocks), dim3(kGemvThreads),
                               chunk_lds, stream, x, packed[s], scales[s], y[s], m, n[s], k, G,
                               chunk, nchunks, RB, kSpliceConsts);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// m = 1 streaming kernel
// ---------------------------------------------------------------------------

constexpr int kGemv1MaxGpl = 8;                 // groups per lane
constexpr int kGemv1DeferRows = 256;            // rows of a wave's deferred results

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

// The matrices of one m = 1 launch: up to kGemv1MaxSegments weight matrices
// that share x and K (one matrix for q4_gemv).  The host splits the waves
// between them in proportion to their rows; wave w of segment s (w counted
// from wave0[s]) owns row quads [w * base + min(w, extra), +base + (w < extra)).
constexpr int kGemv1MaxSegments = 8;
struct Gemv1Segments {
    const uint8_t* packed[kGemv1MaxSegments];
    const uint16_t* scales[kGemv1MaxSegments];
    float* y[kGemv1MaxSegments];
    int64_t n[kGemv1MaxSegments];
    int64_t wave0[kGemv1MaxSegments];
    int64_t waves[kGemv1MaxSegments];
    int64_t base[kGemv1MaxSegments];
    int64_t extra[kGemv1MaxSegments];
    int count;
};
static_assert(kGemv1MaxSegments == Q4_MULTI_MAX, "segment table must hold Q4_MULTI_MAX matrices");

// LPR lanes share a row (RPS = 64 / LPR rows per wave step); lane `sub` owns
// groups sub + LPR * i, i < GPL, of every row, so G = LPR * GPL.  Each wave
// walks its own contiguous rows front to back with PF steps of loads in
// flight.  Refill loads past the wave's last step re-read that last step
// (this wave's own rows, still cached), so every load is unconditional and
// the compiler keeps PF steps outstanding instead of draining the queue; the
// last PF steps are computed after the loop without new loads.
//
// DEFER: each step's results go to a wave-private LDS buffer instead of to y,
// and the wave writes its whole range (RPS * cnt consecutive rows) with
// coalesced 4-byte stores after its last step.  A global store inside the
// pipelined loop shares the in-order vmcnt queue with the loads, so every
// later wait for a step's codes also waits for the store's write-back; with
// the stores after the loop the queue holds loads only.  The host selects
// DEFER when every wave's range fits the buffer (kGemv1DeferRows rows).
//
// TOPK: instead of storing y, every wave keeps the 32 largest (logit, row)
// keys of its rows (q4_topk.hpp): each step's RPS results go to a 64-entry
// wave buffer in LDS, merged into the running list whenever it is full; at
// the end the four lists of a workgroup are merged and written to
// partials[blockIdx.x * 32 .. +32) (idle waves contribute empty lists).
template <int LPR, int GPL, int PF, bool TOPK, bool DEFER>
__global__ __launch_bounds__(kGemvThreads) void gemv1_kernel(
    const uint16_t* __restrict__ x, int K, Gemv1Segments seg, SpliceConsts kc,
    uint64_t* __restrict__ partials) {
    constexpr int RPS = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;
    const int r = lane / LPR;
    const int G = K / 32;
    const int64_t w = (int64_t)blockIdx.x * kGemvWaves +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // this wave's segment (wave-uniform selects over constant indices)
    const uint8_t* packed = seg.packed[0];
    const uint16_t* scales = seg.scales[0];
    float* y = seg.y[0];
    int64_t N = seg.n[0], wave0 = seg.wave0[0], waves = seg.waves[0];
    int64_t base = seg.base[0], extra = seg.extra[0];
#pragma unroll
    for (int i = 1; i < kGemv1MaxSegments; ++i) {
        if (i < seg.count && w >= seg.wave0[i]) {
            packed = seg.packed[i]; scales = seg.scales[i]; y = seg.y[i];
            N = seg.n[i]; wave0 = seg.wave0[i]; waves = seg.waves[i];
            base = seg.base[i]; extra = seg.extra[i];
        }
    }
    const int64_t lw = w - wave0;
    const bool active = lw < waves;
    const int64_t q0 = lw * base + (lw < extra ? lw : extra);
    const int64_t cnt = active ? base + (lw < extra ? 1 : 0) : 0;
    const int64_t row0 = RPS * q0 + r;

    // top-k state: running list (lanes 0..31) and this wave's candidate buffer
    __shared__ uint64_t cand[TOPK ? kGemvWaves : 1][64];
    uint64_t* buf = cand[TOPK ? (threadIdx.x >> 6) : 0];
    // deferred results of this wave's rows (DEFER)
    __shared__ float ydef[DEFER ? kGemvWaves : 1][DEFER ? kGemv1DeferRows : 1];
    float* ybuf = ydef[DEFER ? (threadIdx.x >> 6) : 0];
    uint64_t list = 0;
    int filled = 0;                                   // steps in the buffer
    auto flush = [&]() {
        __builtin_amdgcn_wave_barrier();
        const uint64_t key = lane < filled * RPS ? buf[lane] : 0;
        __builtin_amdgcn_wave_barrier();
        list = topk_merge_batch(list, key, lane);
        filled = 0;
    };
    // result of step f for this lane's row: stored, or offered to the list
    auto emit = [&](float acc, int64_t f) {
        const int64_t row = row0 + RPS * f;
        if (TOPK) {
            if (sub == 0) buf[filled * RPS + r] = row < N ? topk_key(acc, (uint32_t)row) : 0;
            if (++filled == 64 / RPS) flush();
        } else if (DEFER) {
            if (sub == 0) ybuf[RPS * f + r] = acc;
        } else {
            if (sub == 0 && row < N) y[row] = acc;
        }
    };

    // Weight loads are buffer loads from this wave's first row: the wave's
    // base and the step offset are scalars, the lane's offset within a step
    // is fixed, so a step costs no vector address arithmetic (the 64-bit
    // row * stride products it replaced were six quarter-rate VALU
    // instructions per step).  The buffer ends at the segment's row N: the
    // lanes of a partial last quad read zeros there, and their results are
    // never stored.  The host keeps a wave's range below 2 GiB.
    const int64_t wrow = RPS * q0;
    const int64_t wrows = N > wrow ? N - wrow : 0;
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(packed + wrow * (int64_t)(K / 2)), (short)0,
        (int)(wrows * (K / 2) < 0x7FFFFFFF ? wrows * (K / 2) : 0x7FFFFFFF), kBufferFlags);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(scales + wrow * (int64_t)G), (short)0,
        (int)(wrows * G * 2 < 0x7FFFFFFF ? wrows * G * 2 : 0x7FFFFFFF), kBufferFlags);
    const int poff = r * (K / 2) + 16 * sub;
    const int soff = 2 * (r * G + sub);
    const int last = cnt > 0 ? (int)cnt - 1 : 0;
    u32x4_t rp[PF][GPL];
    uint32_t rs[PF][GPL];
    auto load = [&](int slot, int f) {
        const int fs = f < last ? f : last;      // past the last step: re-read it
        const int pstep = fs * (RPS * (K / 2)), sstep = fs * (RPS * G * 2);
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            rp[slot][i] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(prs, poff + 16 * LPR * i, pstep,
                                                               kBufferNontemporal));
            rs[slot][i] = __builtin_amdgcn_raw_buffer_load_b16(srs, soff + 2 * LPR * i, sstep, 0);
        }
    };
    // Activations: the workgroup stages x in LDS once -- every thread loads
    // at most kXPT of its 16-byte chunks, issued before the weight loads so
    // that waiting for them leaves those in flight -- and each lane reads its
    // GPL groups from there.  Loading them per lane from global memory, four
    // rows of lanes fetching the same values, cost ~3 us per 4B decode step
    // in the small projection launches.  Chunk c of group g sits at slot
    // 5 g + c: one 16-byte pad per group spreads the 16 groups that a read
    // touches over the LDS banks.
    constexpr int kXChunks = 4 * LPR * GPL;                  // K / 8
    constexpr int kXPT = (kXChunks + kGemvThreads - 1) / kGemvThreads;
    // (every x load and store is unconditional -- threads past the last chunk
    // re-load it and store to spare slots -- so that no branch lets the
    // compiler move the loads behind the weight loads, which made it wait
    // for all of them and shortened the loop's prefetch)
    __shared__ u32x4_t xs[kXPT * kGemvThreads / 4 * 5];
    u32x4_t xv[kXPT];
#pragma unroll
    for (int t = 0; t < kXPT; ++t) {
        const int j = (int)threadIdx.x + kGemvThreads * t;
        xv[t] = *reinterpret_cast<const u32x4_t*>(x + 8 * (j < kXChunks ? j : kXChunks - 1));
    }
    __builtin_amdgcn_sched_barrier(0);      // keep them ahead of the weight loads
    // an idle wave (cnt = 0, past its segment's waves) starts at or past row
    // N: its buffers are empty and its loads return zeros it never uses
#pragma unroll
    for (int p = 0; p < PF; ++p) load(p, p);
#pragma unroll
    for (int t = 0; t < kXPT; ++t) {
        const int j = (int)threadIdx.x + kGemvThreads * t;
        xs[j / 4 * 5 + j % 4] = xv[t];
    }
    __builtin_amdgcn_s_waitcnt(kLdsStoresDone);
    barrier_keep_loads();
    if (!TOPK && !active) return;           // the top-k variant's idle waves join the final merge

    // this lane's activations, as fp16 pairs in unpack order
    uint32_t xr[GPL][16];
#pragma unroll
    for (int i = 0; i < GPL; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4_t v = permute_x8(xs[(sub + LPR * i) * 5 + c]);
#pragma unroll
            for (int e = 0; e < 4; ++e) xr[i][4 * c + e] = v[e];
        }

    // Enter the loop with the first PF steps landed: with them still in
    // flight the compiler's wait at the loop head kept only ~3 loads
    // outstanding in every later step (4B head 54.8 -> 63.6 us).  Waves of
    // PF steps or fewer wait here too: skipping the wait for them, so that
    // each step is computed as soon as it lands, made the 0.8B projection
    // launches (one step per wave) 0.5 us slower.
    __builtin_amdgcn_s_waitcnt(0);

    const uint32_t mask = kc.mask, mask16 = kc.mask16;
    const uint32_t magic = to_vgpr(kc.magic);
    // one step: this lane's GPL groups of its row, scaled and summed
    auto compute = [&](int p) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            float lo = 0.f, hi = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                half2_t l[2], h[2];
                unpack8_split(rp[p][i][c], mask, mask16, magic, l, h);
                lo = __builtin_amdgcn_fdot2(l[0], as_half2(xr[i][4 * c + 0]), lo, false);
                hi = __builtin_amdgcn_fdot2(h[0], as_half2(xr[i][4 * c + 1]), hi, false);
                lo = __builtin_amdgcn_fdot2(l[1], as_half2(xr[i][4 * c + 2]), lo, false);
                hi = __builtin_amdgcn_fdot2(h[1], as_half2(xr[i][4 * c + 3]), hi, false);
            }
            acc = fmaf(half_bits_to_float(rs[p][i]), fmaf(hi, 0.0625f, lo), acc);
        }
        return lanes_sum<LPR>(acc);
    };

    const int steps = (int)cnt;                 // below 2^31: the host bounds a wave's bytes
    int f0 = 0;
    for (; f0 + PF < steps; f0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const float acc = compute(p);
            load(p, f0 + p + PF);
            emit(acc, f0 + p);
        }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        if (f0 + p < steps) {
            const float acc = compute(p);
            emit(acc, f0 + p);
        }
    }
    if constexpr (DEFER) {
        // rows RPS * q0 + i, i < RPS * cnt, are this wave's range, in order;
        // LDS serves one wave's accesses in issue order, so the reads see
        // every write above
        __builtin_amdgcn_wave_barrier();
        const int rows = (int)(RPS * cnt);
        for (int i = lane; i < rows; i += 64) {
            const int64_t row = RPS * q0 + i;
            if (row < N) y[row] = ybuf[i];
        }
    }
    if constexpr (TOPK) {
        // the workgroup's four lists -> one, in partials[blockIdx.x * 32 ..)
        if (filled > 0) flush();
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        if (lane < kTopkList) cand[wave][lane] = list;
        __syncthreads();
        if (wave == 0) {
            // the other lists are sorted already: three bitonic merges
            // (6 stages each) instead of sorting them as batches (~27 each)
#pragma unroll
            for (int v = 1; v < kGemvWaves; ++v)
                list = topk_merge_sorted(list, cand[v][lane & (kTopkList - 1)], lane);
            if (lane < kTopkList) partials[(int64_t)blockIdx.x * kTopkList + lane] = list;
        }
    }
}

// Steps in flight per wave and waves per SIMD of the plain launch, from a
// sweep on the LM heads (all variants bit-identical): at K = 1024 (2 groups
// per lane) four steps x two waves per SIMD, at K = 2560 (5 groups per lane)
// two steps x one wave per SIMD were fastest -- about 10-16 KB of code loads
// in flight per SIMD, split so that one wave's unpacking overlaps the other's
// loads where a step is short.
constexpr int gemv1_prefetch(int gpl) {
    return gpl <= 1 ? 8 : gpl == 2 ? 4 : gpl == 3 ? 3 : 2;
}
constexpr int gemv1_waves_per_simd(int gpl) { return gpl <= 3 ? 2 : 1; }

// Waves per SIMD of a launch over `steps` steps: the table's value, except
// that a second wave per SIMD is only used when every wave still gets two
// steps or more -- with one step per wave the fixed cost of a wave (its
// activation loads, the first load round trip) is not amortised, and one
// wave per SIMD with two steps each was faster (k = 1024, n = 6144: 4.38
// against 4.84 us; from n = 16384 rows at k = 1024 on the two are within 2%).
int gemv1_wps(int gpl, int64_t steps, int cu_count) {
    const int wps = gemv1_waves_per_simd(gpl);
    return wps > 1 && steps < 2 * (int64_t)cu_count * kGemvWaves * wps ? 1 : wps;
}

// Waves of one segment of an m = 1 launch.  Short launches (one or two steps
// per wave) size the waves for equal step counts, ceil(steps / per).  Longer
// ones use every wave they may (max_waves) and the segments share them in
// proportion to their steps -- segment s ends at wave round(W * steps before
// its end / total steps) -- so that every wave gets base or base + 1 steps:
// equal counts had left workgroups off the last CUs (the 0.8B LM head, 31
// steps per wave: 501 of 512 workgroups; 25.1 -> 24.6 us, the fused top-20
// 33.0 -> 32.8 us).  For two steps per wave the equal split was faster even
// where it leaves CUs idle (the 4B attention q/k/v launch, 1,536 steps: 768
// waves on 192 CUs, ~0.5 us faster than 1,024 waves of one or two steps).
int64_t gemv1_segment_waves(int64_t rq_before, int64_t rq, int64_t total_rq, int64_t max_waves,
                            int64_t wave0) {
    const int64_t per = (total_rq + max_waves - 1) / max_waves;
    if (per < 3) return (rq + per - 1) / per;
    const int64_t w_all = max_waves;
    const int64_t end = (w_all * (rq_before + rq) + total_rq / 2) / total_rq;
    int64_t waves = end - wave0;
    if (waves > rq) waves = rq;
    return waves < 1 ? 1 : waves;
}

template <int LPR, int GPL>
hipError_t launch_gemv1_t(const uint16_t* x, int k, int count, const uint8_t* const* packed,
                          const uint16_t* const* scales, float* const* y, const int64_t* n,
                          uint64_t* partials, hipStream_t stream) {
    constexpr int PF = gemv1_prefetch(GPL);
    constexpr int RPS = 64 / LPR;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Gemv1Segments seg = {};
    seg.count = count;
    int64_t total_rq = 0;
    for (int s = 0; s < count; ++s) total_rq += (n[s] + RPS - 1) / RPS;
    const int cu = device_info(dev).cu_count;
    const int64_t max_waves = (int64_t)cu * kGemvWaves * gemv1_wps(GPL, total_rq, cu);
    int64_t wave0 = 0, rq_before = 0;
    for (int s = 0; s < count; ++s) {
        const int64_t rq = (n[s] + RPS - 1) / RPS;
        const int64_t waves = gemv1_segment_waves(rq_before, rq, total_rq, max_waves, wave0);
        rq_before += rq;
        seg.packed[s] = packed[s];
        seg.scales[s] = scales[s];
        seg.y[s] = y[s];
        seg.n[s] = n[s];
        seg.wave0[s] = wave0;
        seg.waves[s] = waves;
        seg.base[s] = rq / waves;
        seg.extra[s] = rq % waves;
        wave0 += waves;
    }
    const int blocks = (int)((wave0 + kGemvWaves - 1) / kGemvWaves);
    // Results wait in LDS until a wave's last step (DEFER) when every wave's
    // range fits the buffer and the launch runs two waves per SIMD (GPL <= 3):
    // bit-identical either way; 0.8B LM head (k = 1024) 24.8 -> 24.2 us,
    // while at k = 2560 (one wave per SIMD, two steps in flight) the 4B LM
    // head and its decode step ran 0.2-0.8 us slower with it.
    int64_t most = 0;
    for (int s = 0; s < count; ++s) {
        const int64_t c = seg.base[s] + (seg.extra[s] > 0 ? 1 : 0);
        most = c > most ? c : most;
    }
    // a wave addresses its rows with 32-bit buffer offsets: its range must
    // stay below 2 GiB (with at least one wave per SIMD that takes a matrix
    // of terabytes, far beyond the device's memory)
    if ((most + 1) * RPS * (int64_t)(k / 2) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    if (partials)
        hipLaunchKernelGGL((gemv1_kernel<LPR, GPL, PF, true, false>), dim3(blocks),
                           dim3(kGemvThreads), 0, stream, x, k, seg, kSpliceConsts, partials);
    else if (gemv1_waves_per_simd(GPL) > 1 && most * RPS <= kGemv1DeferRows)
        hipLaunchKernelGGL((gemv1_kernel<LPR, GPL, PF, false, true>), dim3(blocks),
                           dim3(kGemvThreads), 0, stream, x, k, seg, kSpliceConsts, partials);
    else
        hipLaunchKernelGGL((gemv1_kernel<LPR, GPL, PF, false, false>), dim3(blocks),
                           dim3(kGemvThreads), 0, stream, x, k, seg, kSpliceConsts, partials);
    return hipGetLastError();
}

template <int LPR>
hipError_t launch_gemv1_lpr(const uint16_t* x, int k, int count, const uint8_t* const* packed,
                            const uint16_t* const* scales, float* const* y, const int64_t* n,
                            uint64_t* partials, hipStream_t stream) {
    switch ((k / 32) / LPR) {
        case 1: return launch_gemv1_t<LPR, 1>(x, k, count, packed, scales, y, n, partials, stream);
        case 2: return launch_gemv1_t<LPR, 2>(x, k, count, packed, scales, y, n, partials, stream);
        case 3: return launch_gemv1_t<LPR, 3>(x, k, count, packed, scales, y, n, partials, stream);
        case 4: return launch_gemv1_t<LPR, 4>(x, k, count, packed, scales, y, n, partials, stream);
        case 5: return launch_gemv1_t<LPR, 5>(x, k, count, packed, scales, y, n, partials, stream);
        case 6: return launch_gemv1_t<LPR, 6>(x, k, count, packed, scales, y, n, partials, stream);
        case 7: return launch_gemv1_t<LPR, 7>(x, k, count, packed, scales, y, n, partials, stream);
        default: return launch_gemv1_t<LPR, 8>(x, k, count, packed, scales, y, n, partials, stream);
    }
}

// Lanes per row for the m = 1 kernel, or 0 when k does not fit it.
int gemv1_lanes_per_row(int64_t k) {
    const int64_t G = k / 32;
    if (G % 16 == 0 && G / 16 <= kGemv1MaxGpl) return 16;
    if (G % 8 == 0 && G / 8 <= kGemv1MaxGpl) return 8;
    if (G % 32 == 0 && G / 32 <= kGemv1MaxGpl) return 32;
    return 0;
}

hipError_t launch_gemv1(const uint16_t* x, int k, int count, const uint8_t* const* packed,
                        const uint16_t* const* scales, float* const* y, const int64_t* n,
                        uint64_t* partials, hipStream_t stream) {
    switch (gemv1_lanes_per_row(k)) {
        case 8: return launch_gemv1_lpr<8>(x, k, count, packed, scales, y, n, partials, stream);
        case 16: return launch_gemv1_lpr<16>(x, k, count, packed, scales, y, n, partials, stream);
        default: return launch_gemv1_lpr<32>(x, k, count, packed, scales, y, n, partials, stream);
    }
}

hipError_t launch_gemv_blockdiag(const uint16_t* x, int64_t m, int64_t k, int count,
                                 const uint8_t* const* packed, const uint16_t* const* scales,
                                 float* const* y, const int64_t* n, hipStream_t stream) {
    if (m <= 4) return launch_gemv_t<1>(x, (int)m, (int)k, count, packed, scales, y, n, stream);
    return launch_gemv_t<2>(x, (int)m, (int)k, count, packed, scales, y, n, stream);
}

}  // namespace

hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed,
                       const uint16_t* scales, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
    if (m == 1 && gemv1_lanes_per_row(k) != 0)
        return launch_gemv1(x, (int)k, 1, &packed, &scales, &y, &n, nullptr, stream);
    if (m >= 2 && n <= kGemvTileRows)
        return launch_gemm_small(x, 1, &packed, &scales, &y, &n, m, k, stream);
    return launch_gemv_blockdiag(x, m, k, 1, &packed, &scales, &y, &n, stream);
}

int64_t gemv1_topk_lists(int64_t n, int64_t k, int cu_count) {
    const int lpr = gemv1_lanes_per_row(k);
    if (lpr == 0) return 0;
    // the m = 1 launcher's grid for one matrix of n rows (launch_gemv1_t):
    // waves per SIMD from the groups per lane and the steps, rounded up to
    // whole workgroups
    const int gpl = (int)((k / 32) / lpr);
    const int64_t rq = (n + 64 / lpr - 1) / (64 / lpr);
    const int64_t max_waves = (int64_t)cu_count * kGemvWaves * gemv1_wps(gpl, rq, cu_count);
    const int64_t waves = gemv1_segment_waves(0, rq, rq, max_waves, 0);
    return (waves + kGemvWaves - 1) / kGemvWaves;            // one list per workgroup
}

hipError_t launch_gemv1_topk(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                             int64_t n, int64_t k, uint64_t* partials, hipStream_t stream) {
    float* none = nullptr;
    return launch_gemv1(x, (int)k, 1, &packed, &scales, &none, &n, partials, stream);
}

hipError_t launch_gemv_multi(const uint16_t* x, int64_t m, int64_t k, int count,
                             const uint8_t* const* packed, const uint16_t* const* scales,
                             float* const* y, const int64_t* n, hipStream_t stream) {
    if (m == 1 && gemv1_lanes_per_row(k) != 0)
        return launch_gemv1(x, (int)k, count, packed, scales, y, n, nullptr, stream);
    if (m == 1) return launch_gemv_blockdiag(x, m, k, count, packed, scales, y, n, stream);
    // m >= 2: every matrix takes the kernel q4_gemv takes for it alone (so
    // its result is bit-identical): one launch for those of at most
    // kGemvTileRows rows, one for the rest
    const uint8_t* sp[kFlatMaxSegments];
    const uint16_t* ss[kFlatMaxSegments];
    float* sy[kFlatMaxSegments];
    int64_t sn[kFlatMaxSegments];
    const uint8_t* lp[kFlatMaxSegments];
    const uint16_t* ls[kFlatMaxSegments];
    float* ly[kFlatMaxSegments];
    int64_t ln[kFlatMaxSegments];
    int small = 0, large = 0;
    for (int s = 0; s < count; ++s) {
        if (n[s] <= kGemvTileRows) {
            sp[small] = packed[s]; ss[small] = scales[s]; sy[small] = y[s]; sn[small] = n[s];
            ++small;
        } else {
            lp[large] = packed[s]; ls[large] = scales[s]; ly[large] = y[s]; ln[large] = n[s];
            ++large;
        }
    }
    if (small > 0) {
        const hipError_t e = launch_gemm_small(x, small, sp, ss, sy, sn, m, k, stream);
        if (e != hipSuccess || large == 0) return e;
    }
    return launch_gemv_blockdiag(x, m, k, large, lp, ls, ly, ln, stream);
}

}  // namespace q4
