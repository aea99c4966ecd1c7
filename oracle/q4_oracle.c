/*
 * q4_oracle.c -- plain, slow, CPU reference of the 4-bit symmetric group
 * quantizer and of the quantized matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the GPU library, and the
 * GPU library never calls it.
 *
 * What it follows:
 *   - QORA-4B forum article, section on quantization and memory management,
 *     and the QORA-LLM-0.8B model card, "Weight Format": weights are
 *     quantized to 4 bits, symmetrically, in groups of 32, and dequantized
 *     through a lookup table.
 *   - QORA-LLM-0.8B model card, "AVX-512 SIMD Acceleration" (Q4 GEMV row):
 *     the product looks each 4-bit code up in a 16-entry table.
 *   - The pages fix no bit layout, rounding or scale rule.  The readings used
 *     here (scale = binary16(max|w| / 7), q = clamp(rne(w / s), -8, 7), q = 0
 *     when s == 0, code stored as q + 8 with the even element in the low
 *     nibble, one binary16 scale per group) are the ones the library header
 *     documents; each is pinned by the CPU test suite.
 *
 * Precision: quantization in IEEE fp32 (the definition); the product and its
 * error bound in fp64, where every 32-term group sum of fp16 * small-integer
 * products is exact.
 *
 * Build: gcc -O2 -fPIC -shared -fopenmp -ffp-contract=off (no fast-math).
 */
#include "q4_oracle.h"

#include <float.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* binary16 <-> binary32/64, written from the IEEE 754 encoding.           */
/* ---------------------------------------------------------------------- */

/* Round an fp32 value to the nearest binary16, ties to even.  Overflow
 * (|f| >= 65520) gives infinity; values at or below 2^-25 give zero. */
uint16_t q4o_f32_to_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t bexp = (u >> 23) & 0xFFu;
    uint32_t frac = u & 0x7FFFFFu;

    if (bexp == 0xFFu)                       /* inf or nan */
        return (uint16_t)(sign | 0x7C00u | (frac ? 0x0200u : 0u));
    if (bexp == 0)                           /* fp32 zero or subnormal: < 2^-126 */
        return sign;

    int e = (int)bexp - 127;                 /* value = sig * 2^(e - 23) */
    uint32_t sig = frac | 0x800000u;         /* 24-bit significand */

    if (e > 15)
        return (uint16_t)(sign | 0x7C00u);

    if (e >= -14) {
        /* binary16 normal: keep 11 significant bits */
        uint32_t r = sig >> 13;
        uint32_t rem = sig & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (r & 1u)))
            r++;
        uint32_t he = (uint32_t)(e + 15);
        if (r == 2048u) {                    /* carried into the next binade */
            r = 1024u;
            he++;
        }
        if (he >= 31u)
            return (uint16_t)(sign | 0x7C00u);
        return (uint16_t)(sign | (he << 10) | (r - 1024u));
    }

    /* binary16 subnormal: value = r * 2^-24, r = sig * 2^(e + 1) */
    int shift = -(e + 1);                    /* >= 14 here */
    if (shift > 24)                          /* value < 2^-25: rounds to zero */
        return sign;
    uint32_t r = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (r & 1u)))
        r++;
    return (uint16_t)(sign | r);             /* r == 1024 encodes 2^-14 */
}

double q4o_f16_to_f64(uint16_t h) {
    int neg = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return neg ? -v : v;
}

/* ---------------------------------------------------------------------- */
/* Quantizer                                                               */
/* ---------------------------------------------------------------------- */

/* The 16-entry dequantization table: a stored 4-bit code v stands for the
 * signed level v - 8. */
static const int kLevel[16] = {-8, -7, -6, -5, -4, -3, -2, -1,
                               0,  1,  2,  3,  4,  5,  6,  7};

/* Level of one weight given the group's (widened) scale. */
static int level_of(float w, float s) {
    if (s == 0.0f)
        return 0;                            /* zero-scale group: every level 0 */
    float v = nearbyintf(w / s);             /* fp32 division, ties to even */
    if (v < -8.0f)
        return -8;
    if (v > 7.0f)
        return 7;
    return (int)v;
}

int q4o_quantize(const float* w, int64_t n, int64_t k,
                 uint8_t* packed, uint16_t* scales) {
    if (!w || !packed || !scales)
        return Q4O_ERR_NULL;
    if (n < 1 || k < 32 || k % 32 != 0)
        return Q4O_ERR_SHAPE;
    const int64_t G = k / 32;
    int bad = 0;

#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t j = 0; j < G; ++j) {
            const float* g = w + r * k + 32 * j;
            float amax = 0.0f;
            for (int t = 0; t < 32; ++t) {
                float a = fabsf(g[t]);
                if (!(a <= FLT_MAX))         /* nan or inf */
                    bad = 1;
                if (a > amax)
                    amax = a;
            }
            float ratio = amax / 7.0f;
            uint16_t s16 = q4o_f32_to_f16(ratio);
            if ((s16 & 0x7C00u) == 0x7C00u)  /* scale overflowed binary16 */
                bad = 1;
            float s = (float)q4o_f16_to_f64(s16);
            scales[r * G + j] = s16;

            uint8_t* out = packed + r * (k / 2) + 16 * j;
            for (int t = 0; t < 32; t += 2) {
                int q_even = level_of(g[t], s);
                int q_odd = level_of(g[t + 1], s);
                out[t / 2] = (uint8_t)((q_even + 8) | ((q_odd + 8) << 4));
            }
        }
    }
    return bad ? Q4O_ERR_RANGE : Q4O_OK;
}

/* ---------------------------------------------------------------------- */
/* Product                                                                 */
/* ---------------------------------------------------------------------- */

int q4o_matmul(const uint16_t* x, const uint8_t* packed,
               const uint16_t* scales, int64_t m, int64_t n, int64_t k,
               double* y, double* bound) {
    if (!x || !packed || !scales || !y)
        return Q4O_ERR_NULL;
    if (m < 1 || n < 1 || k < 32 || k % 32 != 0)
        return Q4O_ERR_SHAPE;
    const int64_t G = k / 32;

    double* xd = (double*)malloc((size_t)(m * k) * sizeof(double));
    if (!xd)
        return Q4O_ERR_NOMEM;
    for (int64_t i = 0; i < m * k; ++i)
        xd[i] = q4o_f16_to_f64(x[i]);

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t* row = packed + r * (k / 2);
        for (int64_t i = 0; i < m; ++i) {
            const double* xi = xd + i * k;
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t j = 0; j < G; ++j) {
                double s = q4o_f16_to_f64(scales[r * G + j]);
                double dot = 0.0, dot_abs = 0.0;  /* exact in fp64 */
                for (int t = 0; t < 32; ++t) {
                    int64_t kk = 32 * j + t;
                    uint8_t byte = row[kk / 2];
                    int code = (kk % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
                    double term = xi[kk] * (double)kLevel[code];
                    dot += term;
                    dot_abs += fabs(term);
                }
                acc += s * dot;
                acc_abs += fabs(s) * dot_abs;
            }
            y[i * n + r] = acc;
            if (bound)
                bound[i * n + r] = acc_abs;
        }
    }
    free(xd);
    return Q4O_OK;
}

/* ---------------------------------------------------------------------- */
/* Product with fp16 weights (the pages' other weight format)              */
/* ---------------------------------------------------------------------- */

/* QORA-4B forum article, quantization section (format table: F16 beside
 * Q4) and QORA-LLM-0.8B model card, "AVX-512 SIMD Acceleration" (F16 GEMV
 * row: each fp16 weight widened, then multiply-accumulated).  The plain
 * definition y[i,r] = sum_t x[i,t] * w[r,t], in fp64: every product of two
 * binary16 values is exact there. */
int q4o_matmul_f16(const uint16_t* x, const uint16_t* w, int64_t m, int64_t n,
                   int64_t k, double* y, double* bound) {
    if (!x || !w || !y)
        return Q4O_ERR_NULL;
    if (m < 1 || n < 1 || k < 1)
        return Q4O_ERR_SHAPE;
    double* xd = (double*)malloc((size_t)(m * k) * sizeof(double));
    if (!xd)
        return Q4O_ERR_NOMEM;
    for (int64_t i = 0; i < m * k; ++i)
        xd[i] = q4o_f16_to_f64(x[i]);

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t* row = w + r * k;
        for (int64_t i = 0; i < m; ++i) {
            const double* xrow = xd + i * k;
            double sum = 0.0, sum_abs = 0.0;
            for (int64_t t = 0; t < k; ++t) {
                double prod = xrow[t] * q4o_f16_to_f64(row[t]);
                sum += prod;
                sum_abs += fabs(prod);
            }
            y[i * n + r] = sum;
            if (bound)
                bound[i * n + r] = sum_abs;
        }
    }
    free(xd);
    return Q4O_OK;
}

/* Number of threads the parallel loops above use (1 without OpenMP). */
int q4o_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of later parallel loops (for timing; no effect on
 * any result, which never depends on the split over threads). */
void q4o_set_threads(int threads) {
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
}
