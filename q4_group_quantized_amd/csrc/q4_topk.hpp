// q4_topk.hpp -- wave-level top-32 selection of (logit, row) pairs for the
// LM-head epilogue (greedy decoding picks the largest logit; top-k sampling
// keeps the k largest: QORA-LLM-0.8B model card, CLI options and "Sampling
// Defaults", top_k = 20; the verify step of speculative decoding scores a few
// draft tokens at once: Rai article, speculative decoding section).
//
// A candidate is a 64-bit key that orders like (value, -row): the high word
// maps the fp32 bit pattern onto an unsigned total order (+0 above -0, -inf
// lowest), the low word is ~row, so equal values rank the smaller row first.
// NaN maps to key 0, the same as an empty slot: below every number.
//
// A wave holds its running top-32 sorted descending in lanes 0..31.  A batch
// of 64 new keys (one per lane) is sorted by a bitonic network, its top 32 are
// laid reversed into lanes 32..63 behind the list -- one bitonic sequence --
// and a bitonic merge leaves the new top-32 in lanes 0..31.  Exchanges inside
// 16-lane rows are DPP register moves; only the 16- and 32-lane strides go
// through the LDS crossbar.  The result depends only on the set of keys, so
// it is deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr int kTopkList = 32;               // entries kept per wave

__device__ __forceinline__ uint64_t topk_key(float v, uint32_t row) {
    if (v != v) return 0;
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    const uint32_t hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)hi << 32) | (uint64_t)(~row);
}

__device__ __forceinline__ float topk_value(uint64_t key) {
    if (key == 0) return __builtin_bit_cast(float, 0x7FC00000u);
    const uint32_t hi = (uint32_t)(key >> 32);
    const uint32_t b = (hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi;
    return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ int32_t topk_row(uint64_t key) {
    return key == 0 ? -1 : (int32_t)(~(uint32_t)key);
}

// Key of lane (lane ^ S) for S = 1, 2, 4, 8 (DPP moves inside 16-lane rows:
// quad permutes, and the row / half-row mirrors, which are lane ^ 15 and
// lane ^ 7), S = 16 (ds_swizzle, xor mode inside 32 lanes) and S = 32
// (ds_bpermute).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    return ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
template <int S>
__device__ __forceinline__ uint64_t xor_lane(uint64_t v) {
    if (S == 1) return dpp64<0xB1>(v);                        // quad_perm 1,0,3,2
    if (S == 2) return dpp64<0x4E>(v);                        // quad_perm 2,3,0,1
    if (S == 4) return dpp64<0x1B>(dpp64<0x141>(v));          // (l ^ 7) ^ 3
    if (S == 8) return dpp64<0x141>(dpp64<0x140>(v));         // (l ^ 15) ^ 7
    if (S == 16) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)v, 0x401F);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_swizzle((int)(uint32_t)(v >> 32), 0x401F);
        return ((uint64_t)hi << 32) | lo;
    }
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, 32, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), 32, 64);
    return ((uint64_t)hi << 32) | lo;
}

// One compare-exchange of a bitonic network: lanes at distance S pair up and
// the lane for which `keep_max` holds keeps the larger key.
template <int S>
__device__ __forceinline__ uint64_t cmpx(uint64_t key, bool keep_max) {
    const uint64_t other = xor_lane<S>(key);
    const bool gt = key > other;
    return (gt == keep_max) ? key : other;
}

template <int SIZE, int S>
__device__ __forceinline__ uint64_t sort_stage(uint64_t key, int lane) {
    const bool lower = (lane & S) == 0;
    const bool desc = SIZE == 64 || (lane & SIZE) == 0;
    return cmpx<S>(key, lower == desc);
}

// Sorts one key per lane, descending across the wave (bitonic network).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t key, int lane) {
    key = sort_stage<2, 1>(key, lane);
    key = sort_stage<4, 2>(key, lane);   key = sort_stage<4, 1>(key, lane);
    key = sort_stage<8, 4>(key, lane);   key = sort_stage<8, 2>(key, lane);
    key = sort_stage<8, 1>(key, lane);
    key = sort_stage<16, 8>(key, lane);  key = sort_stage<16, 4>(key, lane);
    key = sort_stage<16, 2>(key, lane);  key = sort_stage<16, 1>(key, lane);
    key = sort_stage<32, 16>(key, lane); key = sort_stage<32, 8>(key, lane);
    key = sort_stage<32, 4>(key, lane);  key = sort_stage<32, 2>(key, lane);
    key = sort_stage<32, 1>(key, lane);
    key = sort_stage<64, 32>(key, lane); key = sort_stage<64, 16>(key, lane);
    key = sort_stage<64, 8>(key, lane);  key = sort_stage<64, 4>(key, lane);
    key = sort_stage<64, 2>(key, lane);  key = sort_stage<64, 1>(key, lane);
    return key;
}

// Merges two sorted lists held in lanes 0..31 of `a` and of `b` (descending)
// into the top 32 of their union, in lanes 0..31 of the result: b reversed
// behind a is one bitonic sequence, so six exchange stages sort it.
__device__ __forceinline__ uint64_t topk_merge_sorted(uint64_t a, uint64_t b, int lane) {
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

// Merges a batch of 64 keys (any order, one per lane) into the running list
// (lanes 0..31, sorted descending); returns the new list in lanes 0..31.  A
// batch with no key above the list's last entry cannot change the list and is
// skipped (the decision is wave-uniform).
__device__ __forceinline__ uint64_t topk_merge_batch(uint64_t list, uint64_t batch, int lane) {
    const uint32_t last_lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)list, kTopkList - 1);
    const uint32_t last_hi =
        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(list >> 32), kTopkList - 1);
    const uint64_t last = ((uint64_t)last_hi << 32) | last_lo;
    if (__builtin_amdgcn_ballot_w64(batch > last) == 0) return list;
    // the batch's top 32, sorted, merged like a list
    return topk_merge_sorted(list, wave_sort_desc(batch, lane), lane);
}

}  // namespace q4
