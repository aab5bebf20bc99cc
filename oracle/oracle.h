/*
 * CPU oracle for the fused-dequant quantized product y[N x M] = x[N x K] . W^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load this library.  It shares no code with the HIP library:
 * its own fp16 / e4m3 / e2m1 decoders, its own superblock unpackers, plain loops,
 * fp64 sums in sequential k order.  Nothing on the product path may call it.
 *
 * Type codes: 12 = Q4_K, 13 = Q5_K, 14 = Q6_K (the GGML type numbers the decode
 * GEMV page's typed-kernel template arguments <12>, <12,12>, <12,12,14> use),
 * 1001 = NVFP4 and 1002 = block-scaled FP8 (this library's own codes; the pages
 * give none).
 *
 * Return values: 0 on success, -1 on a bad argument.
 */
#ifndef QG_ORACLE_H
#define QG_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact decoders (for the pin tests). */
double oracle_fp16(uint16_t bits);
double oracle_e4m3(uint8_t bits);
double oracle_e2m1(uint8_t code);
double oracle_bf16(uint16_t bits);

/* Bytes of one stored row (NVFP4: codes only). -1 if the type or k is invalid. */
int64_t oracle_row_bytes(int32_t type, int64_t k);

/* Dequantize rows [r0, r0+nr) of an m x k weight to fp32 (the exact value rounded
 * once, to nearest even), out is [nr][k]. */
int oracle_dequant(int32_t type, const uint8_t *data, const uint8_t *scales,
                   int64_t m, int64_t k, int64_t r0, int64_t nr, float *out);

/* The same rows as exact values in fp64 (every weight of the four formats is
 * exactly representable there). */
int oracle_dequant64(int32_t type, const uint8_t *data, const uint8_t *scales,
                     int64_t m, int64_t k, int64_t r0, int64_t nr, double *out);

/*
 * y[t][i] = sum_k w[rows[i]][k] * x[t][k]  (fp64, sequential k),
 * a[t][i] = sum_k |w[rows[i]][k]| * |x[t][k]|.
 * x is fp16 bits [n][k]; y and a are [n][nrows].  rows == NULL means all m rows
 * in order (nrows must then equal m).  nthreads <= 0 uses the OpenMP default.
 */
int oracle_gemm(int32_t type, const uint8_t *data, const uint8_t *scales,
                int64_t m, int64_t k, const uint16_t *x, int64_t n,
                const int64_t *rows, int64_t nrows, double *y, double *a,
                int32_t nthreads);

/* Threads the last oracle_gemm call ran with. */
int32_t oracle_last_threads(void);

/* silu(g) * u in fp64, elementwise over len values. */
void oracle_swiglu(const double *g, const double *u, int64_t len, double *out);

#ifdef __cplusplus
}
#endif
#endif
