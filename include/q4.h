/*
 * q4.h -- C ABI of the MI355X (gfx950) weight-only 4-bit group-quantized
 * matrix-vector / matrix-matrix product and of the quantizer that feeds it.
 *
 * The method: weights are quantized symmetrically to 4 bits in groups of 32
 * consecutive input elements, and dequantized through a 16-entry lookup
 * table inside the product (QORA-4B forum article, section on quantization
 * and memory management; QORA-LLM-0.8B model card, "Weight Format" and the
 * Q4 GEMV row of "AVX-512 SIMD Acceleration").  The pages name the scheme but
 * fix no bit layout; the layout below is the one this library defines.
 *
 * Data layout (all tensors dense, row-major, no strides):
 *   W       fp32    [n, k]      weights, one output feature per row
 *   packed  uint8   [n, k/2]    byte i of row r holds element 2i of the row in
 *                               its low nibble and element 2i+1 in its high
 *                               nibble, each stored as q + 8 (0..15)
 *   scales  fp16    [n, k/32]   one scale per group of 32 elements, carried
 *                               as raw IEEE binary16 bit patterns (uint16_t)
 *   x       fp16    [m, k]      activations, raw binary16 bits
 *   y       fp32    [m, n]      y[i][r] = sum_j s[r][j] * sum_t x[i][32j+t] * q[r][32j+t]
 *
 * Quantization of one group g (32 fp32 values w):
 *   amax = max |w|                       (exact)
 *   s    = fp16_rne( amax / 7.0f )       (IEEE fp32 division, then round to
 *                                         nearest-even binary16)
 *   q    = 0                             if s == 0
 *          clamp(rne(w / float(s)), -8, 7) otherwise (IEEE fp32 division of w
 *                                         by the stored fp16 scale widened to
 *                                         fp32, rounded half to even)
 * The result is unique: every implementation must produce identical bytes.
 *
 * Common argument rules for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or keeps them after the call returns.  Only
 *     q4_gemv_topk takes a workspace, which the caller provides.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Work is enqueued asynchronously; the caller keeps inputs alive and
 *     unmodified until the stream has completed it.  Outputs are overwritten
 *     (never accumulated into) and must not alias any input.
 *   - Shapes: n >= 1, k >= 32, k % 32 == 0, n <= 2^31 - 1, k <= 2^24, and
 *     n * k <= 2^40; otherwise Q4_ERR_SHAPE.
 *   - Alignment: x, packed and w 16-byte aligned, y 4-byte aligned,
 *     scales 2-byte aligned; otherwise Q4_ERR_ALIGN.
 *   - Validation happens on the host, synchronously, before anything is
 *     enqueued; on any error nothing is launched.  A launch failure reported
 *     by the HIP runtime maps to Q4_ERR_LAUNCH.  Faults raised asynchronously
 *     by the device surface at the caller's next synchronisation, as with any
 *     HIP work.  No C++ exception and no abort crosses this interface.
 *   - Results are deterministic: no atomics, bit-identical from run to run.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4_ABI_VERSION 7
#define Q4_GROUP 32
#define Q4_MULTI_MAX 8
#define Q4_TOPK_MAX 32
#define Q4_NOALLOC_SCRATCH_BYTES (16u << 20)   /* q4_gemv_topk_noalloc's buffer */

typedef enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,    /* a required pointer is NULL                        */
    Q4_ERR_SHAPE = 2,   /* m, n or k outside the documented ranges            */
    Q4_ERR_ALIGN = 3,   /* a pointer breaks the alignment rule                */
    Q4_ERR_LAUNCH = 4,  /* the HIP runtime refused or failed the launch       */
    Q4_ERR_DEVICE = 5,  /* no usable gfx950 device is current                 */
    Q4_ERR_WORKSPACE = 6, /* workspace NULL, smaller than required or not 256-B aligned */
    Q4_ERR_TOO_LARGE = 7  /* q4_gemv_topk_noalloc: scratch need above Q4_NOALLOC_SCRATCH_BYTES */
} q4_status;

/* Version of this interface; equals Q4_ABI_VERSION of the built library. */
int q4_abi_version(void);

/* Static, NUL-terminated English name of a status code (never NULL). */
const char* q4_status_str(q4_status status);

/*
 * q4_quantize -- symmetric 4-bit group quantization of a weight matrix.
 * Follows the Q4 format the QORA pages describe (4-bit, symmetric, groups of
 * 32) with the bit-level rules stated at the top of this header.
 *   w       [in]  fp32 [n, k], device
 *   packed  [out] uint8 [n, k/2], device
 *   scales  [out] fp16 bits [n, k/32], device
 * Precondition (not checked, outside the contract): every w is finite and
 * |w| < 7 * 65520, so that every scale is a finite binary16.
 */
q4_status q4_quantize(const float* w, uint8_t* packed, uint16_t* scales,
                      int64_t n, int64_t k, void* stream);

/*
 * q4_gemv -- decode-time product y = x * dequant(W)^T for 1 <= m <= 8 rows of
 * activations (one token, or a handful such as a speculative-verify batch).
 * This is the Q4 GEMV that the QORA engines run for every projection and for
 * the 248,320-row LM head (QORA-LLM-0.8B model card, "AVX-512 SIMD
 * Acceleration" and "Weight Format"; QORA-4B article, quantization section).
 *   x       [in]  fp16 bits [m, k], device
 *   packed  [in]  uint8 [n, k/2], device (layout above)
 *   scales  [in]  fp16 bits [n, k/32], device
 *   y       [out] fp32 [m, n], device
 * m outside 1..8 -> Q4_ERR_SHAPE (use q4_gemm).
 * Accuracy: fp16 x times exact integers, fp32 accumulation, group scale
 * applied in fp32 after each 32-element dot product.
 * At m >= 2 a matrix of at most 4096 rows is computed by q4_gemm's
 * small-batch kernel (16-row tiles; its waves split k), which finishes such
 * matrices sooner than the streaming GEMV; the kernel, and so the order of
 * the fp32 sums, depends only on m, n and k.
 */
q4_status q4_gemv(const uint16_t* x, const uint8_t* packed,
                  const uint16_t* scales, float* y,
                  int64_t m, int64_t n, int64_t k, void* stream);

/*
 * q4_gemv_multi -- several decode products over the SAME activations in one
 * call: y_i = x * dequant(W_i)^T for i < count, every W_i with the same k.
 * Projections that read one input are such a set: the fused gate+up GEMV of
 * the QORA-LLM-0.8B card ("AVX-512 SIMD Acceleration"), and the q/k/v
 * projections of one layer input in the hybrid DeltaNet/attention stack
 * ("Architecture" table of the same card).  One launch serves the whole set
 * at m = 1; at m >= 2 one launch serves the matrices of at most 4096 rows
 * (q4_gemv's small-batch kernel) and one the others (at k above 7680, or
 * 15360 for m <= 4, where the activations no longer fit the LDS at once, one
 * launch per matrix), so the fixed cost of a kernel is paid once per kind,
 * not per matrix.
 *   x       [in]  fp16 bits [m, k], device, 1 <= m <= 8
 *   count         number of matrices, 1 .. Q4_MULTI_MAX
 *   packed  [in]  HOST array of count device pointers, uint8 [n[i], k/2]
 *   scales  [in]  HOST array of count device pointers, fp16 bits [n[i], k/32]
 *   y       [out] HOST array of count device pointers, fp32 [m, n[i]]
 *   n       [in]  HOST array of count row counts
 * The host arrays are read during the call only.  Every matrix follows the
 * shape and alignment rules of q4_gemv; count outside 1..Q4_MULTI_MAX ->
 * Q4_ERR_SHAPE; a NULL array or element -> Q4_ERR_NULL.  The outputs must
 * not overlap each other or any input (not checked).  Each y[i] is
 * bit-identical to what q4_gemv returns for matrix i alone.
 */
q4_status q4_gemv_multi(const uint16_t* x, int64_t m, int64_t k, int32_t count,
                        const uint8_t* const* packed, const uint16_t* const* scales,
                        float* const* y, const int64_t* n, void* stream);

/*
 * q4_gemv_f16 -- decode-time product with fp16 weights, the second weight
 * format of the QORA engines (QORA-4B article, quantization section, format
 * table: F16 beside Q4; QORA-LLM-0.8B model card, "AVX-512 SIMD
 * Acceleration", F16 GEMV row).  y[i][r] = sum_t x[i][t] * w[r][t].
 *   x       [in]  fp16 bits [m, k], device, 1 <= m <= 8
 *   w       [in]  fp16 bits [n, k], device (one output feature per row)
 *   y       [out] fp32 [m, n], device
 * Shape and alignment rules as above (k % 32 == 0 here too; w 16-byte
 * aligned like x); m outside 1..8 -> Q4_ERR_SHAPE.
 * Accuracy: products of two fp16 values are exact in fp32; fp32
 * accumulation; the bound |y - y_ref| <= 1e-3 * sum|x * w| + 1e-6 holds.
 */
q4_status q4_gemv_f16(const uint16_t* x, const uint16_t* w, float* y,
                      int64_t m, int64_t n, int64_t k, void* stream);

/*
 * q4_gemm_f16 -- prefill product with fp16 weights: q4_gemv_f16's arguments
 * and semantics for any m in 1 .. 2^31-1 (m <= 8 runs the decode kernel),
 * the batched prefill of the QORA-4B article's GPU section over its F16
 * weight format (quantization section, format table).
 *   x       [in]  fp16 bits [m, k], device, 16-byte aligned
 *   w       [in]  fp16 bits [n, k], device, 16-byte aligned
 *   y       [out] fp32 [m, n], device, 4-byte aligned
 * k % 32 == 0; m * k and m * n within the element limit of q4_gemm, else
 * Q4_ERR_SHAPE.  Accuracy as q4_gemv_f16 (exact products, fp32 sums); the
 * result is deterministic for a given (m, n, k).
 */
q4_status q4_gemm_f16(const uint16_t* x, const uint16_t* w, float* y,
                      int64_t m, int64_t n, int64_t k, void* stream);

/*
 * q4_gemv_topk -- the LM-head product followed by its decoding epilogue: for
 * every token the topk largest logits y[i][r] (r < n) and their rows, without
 * returning the logits.  Greedy decoding takes topk = 1; top-k sampling keeps
 * the k best candidates (QORA-LLM-0.8B model card, CLI options and "Sampling
 * Defaults", top_k = 20); m up to 8 covers the verify batch of speculative
 * decoding (Rai article, speculative decoding section).  The logits are those
 * q4_gemv computes, bit for bit.
 *   x, packed, scales, m, n, k: as q4_gemv (1 <= m <= 8, n <= 2^31 - 2)
 *   topk          1 .. min(Q4_TOPK_MAX, n)
 *   values  [out] fp32 [m, topk], device: largest first
 *   rows    [out] int32 [m, topk], device: the row (vocabulary id) of each
 *   workspace     device scratch of at least q4_gemv_topk_workspace_size(m,
 *                 n, k) bytes, 256-byte aligned, caller-owned; its contents
 *                 are overwritten; calls that share one workspace must not
 *                 overlap in time
 * Order: by value, larger first; equal values by row, smaller first (+0 ranks
 * above -0).  NaN logits rank below every number; a slot that no number
 * fills reports NaN and row -1.  Deterministic.
 * Errors: as q4_gemv; topk out of range -> Q4_ERR_SHAPE; workspace NULL, too
 * small or misaligned -> Q4_ERR_WORKSPACE.
 */
size_t q4_gemv_topk_workspace_size(int64_t m, int64_t n, int64_t k);
q4_status q4_gemv_topk(const uint16_t* x, const uint8_t* packed,
                       const uint16_t* scales, int64_t m, int64_t n, int64_t k,
                       int32_t topk, float* values, int32_t* rows,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * q4_gemv_topk_noalloc -- q4_gemv_topk for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same kernels and
 * bit-identical results as q4_gemv_topk; the scratch comes from a buffer of
 * Q4_NOALLOC_SCRATCH_BYTES (16 MiB) that the library keeps on every device it
 * runs on until the process ends.  The call allocates and frees nothing; its
 * first call on a device looks that device's buffer up (hipGetSymbolAddress).
 *   Arguments as q4_gemv_topk, without workspace and workspace_bytes.
 * Errors: as q4_gemv_topk; a problem whose workspace
 * (q4_gemv_topk_workspace_size) exceeds Q4_NOALLOC_SCRATCH_BYTES ->
 * Q4_ERR_TOO_LARGE (the 248,320-row LM head fits at every m <= 8), and
 * nothing is launched.
 * All calls on one device share its buffer: calls that overlap in time on
 * one device (several streams or host threads) race and must be serialised
 * by the caller.  No part of the buffer needs clearing between calls.
 */
q4_status q4_gemv_topk_noalloc(const uint16_t* x, const uint8_t* packed,
                               const uint16_t* scales, int64_t m, int64_t n, int64_t k,
                               int32_t topk, float* values, int32_t* rows, void* stream);

/*
 * q4_gemm -- prefill product, same arguments and semantics as q4_gemv, for
 * any m in 1 .. 2^31-1 (tuned for m >= 16): all projections of a token batch
 * computed at once, as in the QORA-4B article's GPU prefill section and the
 * batched prefill of the QORA-LLM-0.8B card ("Performance").  m <= 8 runs
 * q4_gemv.  The result is deterministic for a given (m, n, k) on a given
 * device model (the tile shape follows m, n and the number of CUs).
 */
q4_status q4_gemm(const uint16_t* x, const uint8_t* packed,
                  const uint16_t* scales, float* y,
                  int64_t m, int64_t n, int64_t k, void* stream);

/*
 * q4_gemm_multi -- q4_gemm for several matrices over the same token batch in
 * one launch: all projections that read one input during prefill (QORA-4B
 * article, GPU prefill section: the projections of a token batch computed
 * together on the GPU).  Arguments as q4_gemv_multi, with any m >= 1 (m <= 8
 * takes the q4_gemv_multi path, whose outputs are bit-identical to q4_gemv's).
 * Each y[i] meets q4_gemm's accuracy bound and is deterministic for a given
 * set of shapes; for m > 32 the launch picks its tile shape from the tiles of
 * all its matrices, so y[i] may differ from q4_gemm on matrix i alone in the
 * last bits (the order of the fp32 sums follows the tile shape).
 */
q4_status q4_gemm_multi(const uint16_t* x, int64_t m, int64_t k, int32_t count,
                        const uint8_t* const* packed, const uint16_t* const* scales,
                        float* const* y, const int64_t* n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
