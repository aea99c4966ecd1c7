// q4_topk.hip -- the LM-head epilogue: the topk largest logits per token and
// their rows, without handing the logits back to the caller.
//
// m = 1 (greedy decoding, top-k sampling: QORA-LLM-0.8B model card, CLI
// options and "Sampling Defaults"): the streaming GEMV itself keeps each
// wave's top-32 (gemv1_kernel<..., TOPK>), so the 248,320 logits never leave
// the chip; merge_kernel below reduces the per-wave lists.  m = 2..8 (the
// verify batch of speculative decoding: Rai article, speculative decoding
// section): the product is written to the workspace, scan_kernel turns every
// slice of a token's logits into a top-32 list, and merge_kernel reduces them.
// Every list is sorted descending.
#include "q4_launch.hpp"
#include "q4_topk.hpp"

namespace q4 {
namespace {

constexpr int kScanBlocks = 64;        // per token
constexpr int kScanWaves = 4;
constexpr int kScanLists = kScanBlocks * kScanWaves;
constexpr int kMergeWaves = 16;

// Token t = blockIdx.x / kScanBlocks; wave v of the token's kScanLists waves
// takes logits [v * slice, (v + 1) * slice) and writes its list to
// partials[(t * lists + v) * 32 ..].
__global__ __launch_bounds__(64 * kScanWaves) void scan_kernel(const float* __restrict__ logits,
                                                               int64_t n, int64_t lists,
                                                               uint64_t* __restrict__ partials) {
    const int lane = threadIdx.x & 63;
    const int64_t t = blockIdx.x / kScanBlocks;
    const int64_t v = (blockIdx.x % kScanBlocks) * kScanWaves +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t slice = (n + kScanLists - 1) / kScanLists;
    const int64_t beg = v * slice;
    const int64_t end = beg + slice < n ? beg + slice : n;
    const float* row = logits + t * n;
    uint64_t list = 0;
    for (int64_t i = beg; i < end; i += 64) {
        const int64_t j = i + lane;
        const uint64_t key = j < end ? topk_key(row[j], (uint32_t)j) : 0;
        list = topk_merge_batch(list, key, lane);
    }
    if (lane < kTopkList) partials[(t * lists + v) * kTopkList + lane] = list;
}

// Merges two sorted lists held in lanes 0..31 of `a` and of `b` (descending)
// into the top 32 of their union, in lanes 0..31 of the result.
__device__ __forceinline__ uint64_t merge_sorted(uint64_t a, uint64_t b, int lane) {
    const uint32_t src = (uint32_t)(63 - lane) * 4u;
    const uint32_t rlo = (uint32_t)__builtin_amdgcn_ds_bpermute((int)src, (int)(uint32_t)b);
    const uint32_t rhi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)src, (int)(uint32_t)(b >> 32));
    uint64_t v = lane < kTopkList ? a : (((uint64_t)rhi << 32) | rlo);
    v = cmpx<32>(v, (lane & 32) == 0);
    v = cmpx<16>(v, (lane & 16) == 0);
    v = cmpx<8>(v, (lane & 8) == 0);
    v = cmpx<4>(v, (lane & 4) == 0);
    v = cmpx<2>(v, (lane & 2) == 0);
    v = cmpx<1>(v, (lane & 1) == 0);
    return v;
}

constexpr int kCandCap = 2048;
constexpr int kCandBatch = 8;         // keys per thread loaded before testing

// One workgroup per token over its lists partials[t * lists .. + lists), each
// sorted descending.
//  1. The lists' first entries (their maxima) are reduced to their top 32;
//     entry topk-1 of that, T, is a key at most the topk-th largest of all,
//     since the topk heads above it are distinct entries.
//  2. Every entry >= T is a candidate (collected in LDS; their order is
//     irrelevant) -- typically little more than topk of them.
//  3. Wave 0 reduces the candidates to the sorted top 32 and writes topk.
// If more than kCandCap entries reach T (many equal logits), every list is
// merged instead.  Both routes give the top-k of the same set: the result is
// unique.
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(
    const uint64_t* __restrict__ partials, int64_t lists, int topk, float* __restrict__ values,
    int32_t* __restrict__ rows) {
    __shared__ uint64_t wave_lists[kMergeWaves][kTopkList];
    __shared__ uint64_t cand[kCandCap];
    __shared__ uint32_t ncand;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t t = blockIdx.x;
    const uint64_t* src = partials + t * lists * kTopkList;
    if (threadIdx.x == 0) ncand = 0;

    // 1. heads: wave wv takes lists wv*64 + lane (+ 1024 j), sorted into its top 32
    uint64_t heads = 0;
    for (int64_t l0 = 64 * wv; l0 < lists; l0 += 64 * kMergeWaves) {
        const int64_t l = l0 + lane;
        heads = topk_merge_batch(heads, l < lists ? src[l * kTopkList] : 0, lane);
    }
    if (lane < kTopkList) wave_lists[wv][lane] = heads;
    __syncthreads();
#pragma unroll 1
    for (int half = kMergeWaves / 2; half > 0; half >>= 1) {      // tree over the waves
        if (wv < half) {
            const uint64_t b = wave_lists[wv + half][lane & 31];
            heads = merge_sorted(heads, b, lane);
        }
        __syncthreads();
        if (wv < half && lane < kTopkList) wave_lists[wv][lane] = heads;
        __syncthreads();
    }
    const uint64_t thr = wave_lists[0][topk - 1];

    // 2. candidates: each thread loads kCandBatch keys before testing any of
    // them, so their global loads are in flight together (one load per
    // iteration waited for every key in turn: ~16 round trips at m = 1)
    const int64_t total = lists * kTopkList;
    constexpr int64_t kStride = 64 * kMergeWaves;
    for (int64_t i0 = threadIdx.x; i0 < total; i0 += kStride * kCandBatch) {
        uint64_t keys[kCandBatch];
#pragma unroll
        for (int b = 0; b < kCandBatch; ++b) {
            const int64_t i = i0 + b * kStride;
            keys[b] = i < total ? src[i] : 0;
        }
#pragma unroll
        for (int b = 0; b < kCandBatch; ++b) {
            if (keys[b] >= thr && keys[b] != 0) {
                const uint32_t pos = atomicAdd(&ncand, 1u);
                if (pos < kCandCap) cand[pos] = keys[b];
            }
        }
    }
    __syncthreads();
    const uint32_t nc = ncand;

    uint64_t best = 0;
    if (nc <= kCandCap) {
        // 3. wave 0 sorts the candidates
        if (wv == 0) {
            for (uint32_t c0 = 0; c0 < nc; c0 += 64) {
                const uint32_t c = c0 + lane;
                best = topk_merge_batch(best, c < nc ? cand[c] : 0, lane);
            }
        }
    } else {
        // many ties at the threshold: merge every list (each wave a share,
        // then a tree over the waves)
        uint64_t list = 0;
        for (int64_t l = wv; l < lists; l += kMergeWaves)
            list = merge_sorted(list, src[l * kTopkList + (lane & 31)], lane);
        __syncthreads();
        if (lane < kTopkList) wave_lists[wv][lane] = list;
        __syncthreads();
#pragma unroll 1
        for (int half = kMergeWaves / 2; half > 0; half >>= 1) {
            if (wv < half) list = merge_sorted(list, wave_lists[wv + half][lane & 31], lane);
            __syncthreads();
            if (wv < half && lane < kTopkList) wave_lists[wv][lane] = list;
            __syncthreads();
        }
        best = list;
    }
    if (wv == 0 && lane < topk) {
        values[t * topk + lane] = topk_value(best);
        rows[t * topk + lane] = topk_row(best);
    }
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

// Workspace: [partial lists: m * lists * 32 keys][logits: m * n fp32, m > 1 or
// k outside the streaming kernel only].
size_t gemv_topk_workspace(int64_t m, int64_t n, int64_t k, int cu_count) {
    const int64_t fused = m == 1 ? gemv1_topk_lists(n, k, cu_count) : 0;
    const int64_t lists = fused > 0 ? fused : kScanLists;
    size_t bytes = align_up((size_t)(m * lists * kTopkList) * sizeof(uint64_t));
    if (fused == 0) bytes += align_up((size_t)(m * n) * sizeof(float));
    return bytes;
}

hipError_t launch_gemv_topk(const uint16_t* x, const uint8_t* packed, const uint16_t* scales,
                            int64_t m, int64_t n, int64_t k, int topk, float* values,
                            int32_t* rows, void* workspace, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int cu = device_info(dev).cu_count;
    uint64_t* partials = static_cast<uint64_t*>(workspace);
    const int64_t fused = m == 1 ? gemv1_topk_lists(n, k, cu) : 0;
    int64_t lists;
    if (fused > 0) {
        lists = fused;
        e = launch_gemv1_topk(x, packed, scales, n, k, partials, stream);
    } else {
        lists = kScanLists;
        float* logits = reinterpret_cast<float*>(
            static_cast<unsigned char*>(workspace) +
            align_up((size_t)(m * lists * kTopkList) * sizeof(uint64_t)));
        e = launch_gemm(x, packed, scales, logits, m, n, k, stream);
        if (e == hipSuccess) {
            hipLaunchKernelGGL(scan_kernel, dim3((unsigned)(m * kScanBlocks)),
                               dim3(64 * kScanWaves), 0, stream, logits, n, lists, partials);
            e = hipGetLastError();
        }
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)m), dim3(64 * kMergeWaves), 0, stream,
                       partials, lists, topk, values, rows);
    return hipGetLastError();
}

}  // namespace q4
