// q4_device.hpp -- device-side building blocks shared by the gfx950 kernels.
//
// The 16-entry dequantization table (QORA-LLM-0.8B model card, "AVX-512 SIMD
// Acceleration", Q4 GEMV row; QORA-4B article, quantization section) maps a
// stored 4-bit code v to the level v - 8.  On gfx950 the table is not a memory
// lookup: a code is spliced into the low mantissa bits of the binary16
// constant 1024.0 (bit pattern 0x6400), which gives exactly 1024 + v, and one
// packed fp16 subtraction of 1032 yields v - 8, exact, for two codes at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr uint32_t kNibblePairMask = 0x000F000Fu;
constexpr uint32_t kMagic1024x2 = 0x64006400u;   // two binary16 1024.0

__device__ __forceinline__ half2_t as_half2(uint32_t u) {
    return __builtin_bit_cast(half2_t, u);
}
__device__ __forceinline__ uint32_t as_u32(half2_t h) {
    return __builtin_bit_cast(uint32_t, h);
}

// Eight consecutive fp16 activations (as four dwords x0x1, x2x3, x4x5, x6x7)
// reordered to match unpack8_fma: (x0,x4) (x1,x5) (x2,x6) (x3,x7).
__device__ __forceinline__ u32x4_t permute_x8(u32x4_t d) {
    u32x4_t r;
    r[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
    return r;
}

// Constants of the nibble splice, passed to the kernels as an argument.
// gfx9 VOP3 encodings cannot carry two literal constants, so with literals
// the compiler splits (d & mask) | magic into two instructions; values the
// optimizer cannot see are kept in registers and give one v_and_or_b32.
// (No inline asm anywhere: it would make the compiler reserve AGPRs and route
// every MFMA result through them.)
struct SpliceConsts {
    uint32_t mask;       // kNibblePairMask
    uint32_t magic;      // kMagic1024x2
    uint32_t sel[4];     // byte selectors of unpack8_natural
    uint32_t mask16;     // kNibblePairMask16
};
constexpr uint32_t kNibblePairMask16 = 0x00F000F0u;
constexpr SpliceConsts kSpliceConsts = {kNibblePairMask, kMagic1024x2,
                                        {0x0C040C00u, 0x0C050C01u, 0x0C060C02u, 0x0C070C03u},
                                        kNibblePairMask16};

// A kernel-argument value copied into a VGPR (identity DPP move): with the
// mask in an SGPR and the magic in a VGPR the splice is one v_and_or_b32
// (one scalar operand per VOP3).
__device__ __forceinline__ uint32_t to_vgpr(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xE4, 0xF, 0xF, false);
}

// The same table lookup as unpack8_fma, returned as four fp16 pairs
// (e0,e4) (e1,e5) (e2,e6) (e3,e7) for v_dot2_f32_f16.  mask and magic are
// kNibblePairMask and kMagic1024x2 held in registers by the caller.
__device__ __forceinline__ void unpack8_pairs(uint32_t d, uint32_t mask, uint32_t magic,
                                              half2_t (&h)[4]) {
    const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    h[0] = as_half2((d & mask) | magic) + bias;
    h[1] = as_half2(((d >> 4) & mask) | magic) + bias;
    h[2] = as_half2(((d >> 8) & mask) | magic) + bias;
    h[3] = as_half2(((d >> 12) & mask) | magic) + bias;
}

// Eight codes of one packed dword -> eight exact fp16 levels, for an MFMA
// operand.  Dword bits: code of element e (0..7) sits at bits 4e..4e+3.
// Output order (lo half, hi half) per register: (e0,e4) (e1,e5) (e2,e6)
// (e3,e7), i.e. position v of the 8-vector holds element (v >> 1) + 4 (v & 1)
// (activations are permuted to match with permute_x8).
// Codes at bits 0..3 of a byte are spliced into 1024.0 and take -1032; codes
// at bits 4..7 are spliced where they stand (1024 + 16 v) and one fp16 fma
// with 1/16 and -72 gives v - 8 -- exact, since every intermediate is a small
// integer or an exact multiple -- so the dword needs one shift, four
// and-or splices and four packed fp16 operations.  mask, mask16 and magic are
// kNibblePairMask, kNibblePairMask16 and kMagic1024x2 held in registers.
__device__ __forceinline__ half8_t unpack8_fma(uint32_t d, uint32_t mask, uint32_t mask16,
                                               uint32_t magic) {
    const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const half2_t bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t d8 = d >> 8;
    const half2_t h0 = as_half2((d & mask) | magic) + bias;
    const half2_t h1 = __builtin_elementwise_fma(as_half2((d & mask16) | magic), sixteenth, bias16);
    const half2_t h2 = as_half2((d8 & mask) | magic) + bias;
    const half2_t h3 = __builtin_elementwise_fma(as_half2((d8 & mask16) | magic), sixteenth, bias16);
    half8_t r;
    r[0] = h0[0]; r[1] = h0[1];
    r[2] = h1[0]; r[3] = h1[1];
    r[4] = h2[0]; r[5] = h2[1];
    r[6] = h3[0]; r[7] = h3[1];
    return r;
}

// The table lookup with one shift fewer, for v_dot2_f32_f16 with two sums.
// Codes at bits 4..7 of a byte are spliced where they stand: bits 4..7 of the
// mantissa of 1024.0 weigh 16 each, so (d & 0x00F000F0) | 0x64006400 is
// 1024 + 16 v, and subtracting 1152 leaves 16 (v - 8), exact.  Codes at bits
// 0..3 give v - 8 as in unpack8_pairs.  Output, as (lo half, hi half) pairs:
//   lo[0] = (e0, e4) levels        hi[0] = 16 x (e1, e5) levels
//   lo[1] = (e2, e6) levels        hi[1] = 16 x (e3, e7) levels
// The caller sums lo and hi products separately and forms lo + hi / 16, which
// is exact scaling, so every product stays the exact x * level product.
__device__ __forceinline__ void unpack8_split(uint32_t d, uint32_t mask, uint32_t mask16,
                                              uint32_t magic, half2_t (&lo)[2],
                                              half2_t (&hi)[2]) {
    const half2_t bias1 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t bias16 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t d8 = d >> 8;
    lo[0] = as_half2((d & mask) | magic) + bias1;
    hi[0] = as_half2((d & mask16) | magic) + bias16;
    lo[1] = as_half2((d8 & mask) | magic) + bias1;
    hi[1] = as_half2((d8 & mask16) | magic) + bias16;
}

// The table lookup in natural element order, for operands whose activations
// are used as stored: output fp16 v = level of element v (v = 0..7).
// sel[i] = 0x0C040C00 + i * 0x00010001 picks byte i of d into the low half
// and byte i of d >> 4 into the high half; the mask keeps one code per half.
__device__ __forceinline__ half8_t unpack8_natural(uint32_t d, uint32_t mask, uint32_t magic,
                                                   const uint32_t (&sel)[4]) {
    const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const uint32_t u = d >> 4;
    half8_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t h = as_half2((__builtin_amdgcn_perm(u, d, sel[i]) & mask) | magic) + bias;
        r[2 * i] = h[0];
        r[2 * i + 1] = h[1];
    }
    return r;
}

// Sum over the 16 lanes of each DPP row (lanes 16r .. 16r+15); every lane of
// the row receives the total.  Rotations by 8, 4, 2, 1 within the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
    return v;
}

// s_waitcnt operand that waits for this wave's LDS operations only (lgkmcnt
// 0; vmcnt and expcnt at their maxima): gfx9 encoding, vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int kLdsStoresDone = 0xC07F;

// Workgroup barrier that leaves outstanding global loads in flight
// (__syncthreads() also fences memory, which drains every pending load).
// The signal fences only stop the compiler from moving memory accesses across
// it.  Callers first wait themselves for the data other waves will read:
// vmcnt for direct-to-LDS loads, lgkmcnt for LDS stores.
__device__ __forceinline__ void barrier_keep_loads() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Buffer resources for raw (untyped, byte-addressed) buffer loads: word 3 of
// a gfx9 descriptor with a non-zero data format (32-bit) and no swizzle or
// thread-id addressing, and the cache-policy operand that marks a load
// non-temporal (printed as "nt").  A raw buffer load at an offset at or past
// the descriptor's byte count returns zero without touching memory.
constexpr int kBufferFlags = 0x00020000;
constexpr int kBufferNontemporal = 2;

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

}  // namespace q4
