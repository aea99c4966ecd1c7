/*
 * q4_oracle.h -- CPU reference of the 4-bit symmetric group quantizer and of
 * the quantized product.  TEST INFRASTRUCTURE ONLY: used by the test suite,
 * the smoke check and the benchmark's CPU-baseline leg, never by the GPU
 * library (which shares nothing with it).
 */
#ifndef Q4_ORACLE_H
#define Q4_ORACLE_H

#include <stdint.h>

#define Q4O_OK 0
#define Q4O_ERR_NULL 1
#define Q4O_ERR_SHAPE 2
#define Q4O_ERR_RANGE 3   /* non-finite weight, or a scale that overflows binary16 */
#define Q4O_ERR_NOMEM 4

uint16_t q4o_f32_to_f16(float f);
double q4o_f16_to_f64(uint16_t h);

/* w fp32 [n,k] -> packed uint8 [n,k/2], scales binary16 bits [n,k/32].
 * Outputs are written even when Q4O_ERR_RANGE is returned. */
int q4o_quantize(const float* w, int64_t n, int64_t k,
                 uint8_t* packed, uint16_t* scales);

/* y[i,r] = sum_j s[r,j] * sum_t x[i,32j+t] * level(code[r,32j+t]) in fp64,
 * bound[i,r] = sum_j |s[r,j]| * sum_t |x * level| (may be NULL).
 * x binary16 bits [m,k]; y, bound fp64 [m,n]. */
int q4o_matmul(const uint16_t* x, const uint8_t* packed,
               const uint16_t* scales, int64_t m, int64_t n, int64_t k,
               double* y, double* bound);

/* y[i,r] = sum_t x[i,t] * w[r,t] in fp64, bound[i,r] = sum_t |x[i,t] * w[r,t]|
 * (may be NULL).  x binary16 bits [m,k], w binary16 bits [n,k]. */
int q4o_matmul_f16(const uint16_t* x, const uint16_t* w, int64_t m, int64_t n,
                   int64_t k, double* y, double* bound);

/* Threads used by the parallel loops. */
int q4o_threads(void);

/* Thread count of later parallel loops (results do not depend on it). */
void q4o_set_threads(int threads);

#endif
