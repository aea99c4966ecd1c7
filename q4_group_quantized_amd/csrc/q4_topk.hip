// q4_topk.hip -- the LM-head epilogue: the topk largest logits per token and
// their rows, without handing the logits back to the caller.
//
// m = 1 (greedy decoding, top-k sampling: QORA-LLM-0.8B model card, CLI
// options and "Sampling Defaults"): the streaming GEMV itself keeps each
// wave's top-32 (gemv1_kernel<..., TOPK>), so the 248,320 logits never leave
// the chip; merge_kernel below reduces the per-workgroup lists.  m = 2..8 (the
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

constexpr int kScanDepth = 8;          // batches of 64 logits loaded at once

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Token t = blockIdx.x / kScanBlocks; wave v of the token's kScanLists waves
// takes logits [v * slice, (v + 1) * slice) and writes its list to
// partials[(t * lists + v) * 32 ..].  Only keys above the running list's last
// entry (0 until it holds 32) can enter it: those are appended to a wave
// buffer in LDS and merged 64 at a time.  Over a slice of s logits about
// 32 ln(s / 32) keys ever pass (the i-th one seen enters the running top 32
// with probability 32 / i), so most batches of 64 cost a compare and a ballot
// instead of a 64-key sort (one sort per batch took 23.5 us for 8 x 248,320
// logits).
__global__ __launch_bounds__(64 * kScanWaves) void scan_kernel(const float* __restrict__ logits,
                                                               int64_t n, int64_t lists,
                                                               uint64_t* __restrict__ partials) {
    __shared__ uint64_t buf_s[kScanWaves][128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint64_t* buf = buf_s[wave];
    const int64_t t = blockIdx.x / kScanBlocks;
    const int64_t v = (blockIdx.x % kScanBlocks) * kScanWaves + wave;
    const int64_t slice = (n + kScanLists - 1) / kScanLists;
    const int64_t beg = v * slice;
    const int64_t end = beg + slice < n ? beg + slice : n;
    const float* row = logits + t * n;
    uint64_t list = 0, last = 0;
    uint32_t filled = 0;                          // keys in the buffer (wave-uniform)
    for (int64_t i0 = beg; i0 < end; i0 += 64 * kScanDepth) {
        float val[kScanDepth];
#pragma unroll
        for (int d = 0; d < kScanDepth; ++d) {
            const int64_t j = i0 + 64 * d + lane;
            val[d] = j < end ? row[j] : 0.f;
        }
#pragma unroll
        for (int d = 0; d < kScanDepth; ++d) {
            const int64_t j = i0 + 64 * d + lane;
            const uint64_t key = j < end ? topk_key(val[d], (uint32_t)j) : 0;
            const bool pass = key > last;
            const uint64_t bal = __builtin_amdgcn_ballot_w64(pass);
            if (bal == 0) continue;
            const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (pass) buf[filled + below] = key;
            filled += (uint32_t)__builtin_popcountll(bal);
            if (filled >= 64) {
                __builtin_amdgcn_wave_barrier();
                const uint64_t batch = buf[lane];
                const uint64_t rest = buf[64 + lane];
                __builtin_amdgcn_wave_barrier();
                list = topk_merge_batch(list, batch, lane);
                last = readlane64(list, kTopkList - 1);
                filled -= 64;
                if ((uint32_t)lane < filled) buf[lane] = rest;
                __builtin_amdgcn_wave_barrier();
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    if (filled > 0) list = topk_merge_batch(list, (uint32_t)lane < filled ? buf[lane] : 0, lane);
    if (lane < kTopkList) partials[(t * lists + v) * kTopkList + lane] = list;
}

constexpr int kCandCap = 2048;
constexpr int kHeadCap = 64 * kMergeWaves;   // lists per token at most (heads kept in LDS)

// Appends the passing lanes' items through one LDS counter per wave: `store`
// gets each passing lane's slot.  `pass` may differ between lanes; the call
// must be made by every lane of the wave.
template <typename Store>
__device__ __forceinline__ void wave_append(bool pass, uint32_t* counter, int lane, Store store) {
    const uint64_t bal = __builtin_amdgcn_ballot_w64(pass);
    if (bal == 0) return;
    const int first = (int)__builtin_ctzll(bal);
    uint32_t base = 0;
    if (lane == first) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(bal));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, first);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (pass) store(base + below);
}

// One workgroup per token over its lists partials[t * lists .. + lists), each
// sorted descending.
//  1. Bound: lane l of wave 0 takes the largest head (first entry) of lists
//     l, l + 64, ...; entry topk-1 of those 64 maxima sorted, T, is at most
//     the topk-th largest key overall (topk distinct keys reach it).
//  2. Only a list whose head reaches T can hold a key >= T: those lists
//     (typically about topk of them) are collected, and their entries >= T
//     are the candidates.
//  3. Wave 0 reduces the candidates to the sorted top 32 and writes topk.
// Only the heads and the selected lists are read -- reading every list's 32
// entries into one workgroup was bound by that CU's load bandwidth (7.5 against
// 4.3 us on 501 lists).  If more than kCandCap entries reach T (many equal
// logits), every list is merged instead.  Both routes give the
// top-k of the same set: the result is unique.
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(
    const uint64_t* __restrict__ partials, int64_t lists, int topk, float* __restrict__ values,
    int32_t* __restrict__ rows) {
    __shared__ uint64_t wave_lists[kMergeWaves][kTopkList];
    __shared__ uint64_t heads[kHeadCap];
    __shared__ uint32_t sel[kHeadCap];
    __shared__ uint64_t cand[kCandCap];
    __shared__ uint32_t nsel, ncand;
    __shared__ uint64_t thr_s;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int64_t t = blockIdx.x;
    const uint64_t* src = partials + t * lists * kTopkList;
    if (threadIdx.x == 0) {
        nsel = 0;
        ncand = 0;
    }
    // lists <= kHeadCap (launch_gemv_topk): one head per thread
    if ((int64_t)threadIdx.x < lists) heads[threadIdx.x] = src[(int64_t)threadIdx.x * kTopkList];
    __syncthreads();

    // 1. the bound T
    if (wv == 0) {
        uint64_t hm = 0;
        for (int64_t l = lane; l < lists; l += 64) hm = heads[l] > hm ? heads[l] : hm;
        hm = wave_sort_desc(hm, lane);
        const uint64_t thr = readlane64(hm, topk - 1);
        if (lane == 0) thr_s = thr;
    }
    __syncthreads();
    const uint64_t thr = thr_s;

    // 2. lists whose head reaches T, then their entries that do
    {
        const int64_t l = threadIdx.x;
        const uint64_t h = l < lists ? heads[l] : 0;
        wave_append(h >= thr && h != 0, &nsel, lane, [&](uint32_t pos) { sel[pos] = (uint32_t)l; });
    }
    __syncthreads();
    const uint32_t ns = nsel;                     // <= lists
    for (uint32_t j0 = 0; j0 < ns * kTopkList; j0 += 64 * kMergeWaves) {
        const uint32_t j = j0 + threadIdx.x;
        const uint64_t key =
            j < ns * kTopkList ? src[(int64_t)sel[j / kTopkList] * kTopkList + j % kTopkList] : 0;
        wave_append(key >= thr && key != 0, &ncand, lane, [&](uint32_t pos) {
            if (pos < kCandCap) cand[pos] = key;
        });
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
            list = topk_merge_sorted(list, src[l * kTopkList + (lane & 31)], lane);
        __syncthreads();
        if (lane < kTopkList) wave_lists[wv][lane] = list;
        __syncthreads();
#pragma unroll 1
        for (int half = kMergeWaves / 2; half > 0; half >>= 1) {
            if (wv < half) list = topk_merge_sorted(list, wave_lists[wv + half][lane & 31], lane);
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

// Lists of the streaming m = 1 GEMV's top-k form (one per workgroup), or 0
// where it does not apply (m > 1, k outside that kernel, or more workgroups
// than the merge kernel keeps heads for: then the product, scan and merge
// route serves the call, with kScanLists lists per token).
int64_t fused_topk_lists(int64_t m, int64_t n, int64_t k, int cu_count) {
    const int64_t lists = m == 1 ? gemv1_topk_lists(n, k, cu_count) : 0;
    return lists <= kHeadCap ? lists : 0;
}
static_assert(kScanLists <= kHeadCap, "the merge kernel keeps every list head in LDS");

}  // namespace

// Workspace: [partial lists: m * lists * 32 keys][logits: m * n fp32, m > 1 or
// k outside the streaming kernel only].
size_t gemv_topk_workspace(int64_t m, int64_t n, int64_t k, int cu_count) {
    const int64_t fused = fused_topk_lists(m, n, k, cu_count);
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
    const int64_t fused = fused_topk_lists(m, n, k, cu);
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
