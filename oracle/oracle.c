/*
 * CPU oracle: plain dequantizer + fp64 dot product.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Written for readability, not speed:
 * every weight is decoded element by element straight from its defining formula,
 * then each output is an fp64 sum in increasing k.
 *
 * What is computed, and where it is stated:
 *  - The product y[M] = W[M x K] x[K] (N = 1) and y[N x M] = x[N x K] W^T with
 *    W a GGML K-quant tensor: reflex-llm kernel notes (docs/kernels.md), the
 *    K-quant GEMV section and the batched-GEMM section.
 *  - Q4_K / Q5_K weight value dall * sc[sb] * nibble - dmin * m[sb], 8 sub-blocks
 *    of 32 quants, 6-bit scales/mins read through the packed scale table:
 *    reflex-llm Performance page, Path E ("What worked", scale precompute).
 *  - Q4_K qs laid out as four 32-byte chunks, each chunk feeding one sub-block
 *    from its low nibbles and the next from its high nibbles: kernel notes,
 *    uint32 weight-load section (the lane's chunk index il = lane >> 3 selects
 *    one of four 32-byte qs sub-blocks).
 *  - Superblock sizes 144 B (Q4_K) and 210 B (Q6_K): kernel notes, uint32
 *    section; Performance page, Path C (#29).
 *  - NVFP4: 4-bit e2m1 weights with one e4m3 scale per 16 weights, product exact
 *    in fp16: TandemLLM Kernels page, "NVFP4 matrix products".
 *  - Block-scaled FP8: e4m3 codes with one bf16 scale per 128 x 128 block, read as
 *    stored: TandemLLM Kernels page, "FP8 matrix products".  Codes are [M][K];
 *    the scale layout ([ceil(M/128)][K/128], row-major) is not printed there and is
 *    this file's reading.
 *  Byte layouts inside a superblock are not printed on the pages; this file takes
 *  the public GGML K-quant layout (the plainest reading of "GGML K-quant").
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { T_Q4_K = 12, T_Q5_K = 13, T_Q6_K = 14, T_NVFP4 = 1001, T_FP8 = 1002 };

static int32_t g_last_threads = 1;

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double oracle_fp16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1F;
    int f = bits & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + f / 1024.0, e - 15);
    return sign ? -v : v;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 = NaN, no Inf. */
double oracle_e4m3(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int f = bits & 7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp(f / 8.0, -6);
    else
        v = ldexp(1.0 + f / 8.0, e - 7);
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double oracle_bf16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* subnormal: f * 2^-126 / 128 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + f / 128.0, e - 127);
    return sign ? -v : v;
}

/* OCP E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit. */
double oracle_e2m1(uint8_t code) {
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int f = code & 1;
    double v = (e == 0) ? 0.5 * f : ldexp(1.0 + 0.5 * f, e - 1);
    return sign ? -v : v;
}

int64_t oracle_row_bytes(int32_t type, int64_t k) {
    if (k <= 0) return -1;
    switch (type) {
    case T_Q4_K: return (k % 256) ? -1 : (k / 256) * 144;
    case T_Q5_K: return (k % 256) ? -1 : (k / 256) * 176;
    case T_Q6_K: return (k % 256) ? -1 : (k / 256) * 210;
    case T_NVFP4: return (k % 16) ? -1 : k / 2;
    case T_FP8: return (k % 128) ? -1 : k;
    default: return -1;
    }
}

static double u16_at(const uint8_t *p) { return oracle_fp16((uint16_t)(p[0] | (p[1] << 8))); }

/* The 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes s[]:
 * sub-blocks 0..3 keep their fields in the low six bits of s[j] and s[j+4];
 * sub-blocks 4..7 keep the low four bits in the nibbles of s[j+4] and the top two
 * bits in bits 6..7 of s[j-4] (scale) and s[j] (min). */
static void scale_min_6bit(const uint8_t *s, int j, int *sc, int *mn) {
    if (j < 4) {
        *sc = s[j] & 63;
        *mn = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* One Q4_K (has_high = 0) or Q5_K (has_high = 1) superblock -> its 256 weights,
 * exact (d*sc*q and dmin*mn each have at most 22 significant bits, so their
 * difference is exact in fp64). */
static void dequant_q45(const uint8_t *b, int has_high, double *w) {
    double d = u16_at(b), dmin = u16_at(b + 2);
    const uint8_t *s = b + 4;
    const uint8_t *qh = b + 16;
    const uint8_t *qs = b + (has_high ? 48 : 16);
    for (int p = 0; p < 256; p++) {
        int c = p / 64;          /* 32-byte qs chunk */
        int h = (p / 32) % 2;    /* low (0) or high (1) nibble of the chunk */
        int l = p % 32;          /* byte within the chunk */
        int j = 2 * c + h;       /* sub-block */
        int q = (qs[32 * c + l] >> (4 * h)) & 15;
        if (has_high) q += 16 * ((qh[l] >> j) & 1);
        int sc, mn;
        scale_min_6bit(s, j, &sc, &mn);
        w[p] = d * sc * q - dmin * mn;
    }
}

/* One Q6_K superblock -> its 256 weights d * sc * (q - 32), q 6-bit (exact). */
static void dequant_q6(const uint8_t *b, double *w) {
    const uint8_t *ql = b, *qh = b + 128;
    const int8_t *sc = (const int8_t *)(b + 192);
    double d = u16_at(b + 208);
    for (int p = 0; p < 256; p++) {
        int s = p / 128;           /* 128-weight half */
        int g = (p % 128) / 32;    /* 32-weight group inside the half */
        int l = p % 32;
        int lo = (ql[64 * s + 32 * (g & 1) + l] >> (4 * (g >> 1))) & 15;
        int hi = (qh[32 * s + l] >> (2 * g)) & 3;
        int q = lo | (hi << 4);
        int si = 8 * s + 2 * g + l / 16;
        w[p] = d * sc[si] * (q - 32);
    }
}

/* One NVFP4 row: element k is the low nibble of byte k/2 when k is even. */
static void dequant_nvfp4_row(const uint8_t *codes, const uint8_t *scales, int64_t k, double *w) {
    for (int64_t i = 0; i < k; i++) {
        uint8_t code = (codes[i / 2] >> (4 * (i % 2))) & 15;
        w[i] = oracle_e2m1(code) * oracle_e4m3(scales[i / 16]);
    }
}

/* One FP8 row: e4m3 code k times the bf16 scale of block (r / 128, k / 128);
 * scales are [ceil(m/128)][k/128] little-endian bf16. */
static void dequant_fp8_row(const uint8_t *codes, const uint8_t *scales, int64_t k, int64_t r, double *w) {
    const uint8_t *srow = scales + (r / 128) * (k / 128) * 2;
    for (int64_t i = 0; i < k; i++) {
        const uint8_t *sp = srow + (i / 128) * 2;
        w[i] = oracle_e4m3(codes[i]) * oracle_bf16((uint16_t)(sp[0] | (sp[1] << 8)));
    }
}

/* Row r, exact, in fp64. */
static void dequant_row(int32_t type, const uint8_t *data, const uint8_t *scales,
                        int64_t k, int64_t r, double *w) {
    int64_t rb = oracle_row_bytes(type, k);
    const uint8_t *row = data + r * rb;
    switch (type) {
    case T_Q4_K:
        for (int64_t b = 0; b < k / 256; b++) dequant_q45(row + b * 144, 0, w + b * 256);
        break;
    case T_Q5_K:
        for (int64_t b = 0; b < k / 256; b++) dequant_q45(row + b * 176, 1, w + b * 256);
        break;
    case T_Q6_K:
        for (int64_t b = 0; b < k / 256; b++) dequant_q6(row + b * 210, w + b * 256);
        break;
    case T_NVFP4:
        dequant_nvfp4_row(row, scales + r * (k / 16), k, w);
        break;
    case T_FP8:
        dequant_fp8_row(row, scales, k, r, w);
        break;
    }
}

static int check_args(int32_t type, const uint8_t *data, const uint8_t *scales, int64_t m, int64_t k) {
    if (!data || m < 1 || oracle_row_bytes(type, k) < 0) return -1;
    if ((type == T_NVFP4 || type == T_FP8) && !scales) return -1;
    return 0;
}

/* The fp32 weight is the exact value rounded once (the C conversion rounds to
 * nearest, ties to even). */
int oracle_dequant(int32_t type, const uint8_t *data, const uint8_t *scales,
                   int64_t m, int64_t k, int64_t r0, int64_t nr, float *out) {
    if (check_args(type, data, scales, m, k) || !out || r0 < 0 || nr < 0 || r0 + nr > m) return -1;
    double *w = (double *)malloc(sizeof(double) * k);
    if (!w) return -1;
    for (int64_t i = 0; i < nr; i++) {
        dequant_row(type, data, scales, k, r0 + i, w);
        for (int64_t j = 0; j < k; j++) out[i * k + j] = (float)w[j];
    }
    free(w);
    return 0;
}

int oracle_dequant64(int32_t type, const uint8_t *data, const uint8_t *scales,
                     int64_t m, int64_t k, int64_t r0, int64_t nr, double *out) {
    if (check_args(type, data, scales, m, k) || !out || r0 < 0 || nr < 0 || r0 + nr > m) return -1;
    for (int64_t i = 0; i < nr; i++) dequant_row(type, data, scales, k, r0 + i, out + i * k);
    return 0;
}

int oracle_gemm(int32_t type, const uint8_t *data, const uint8_t *scales,
                int64_t m, int64_t k, const uint16_t *x, int64_t n,
                const int64_t *rows, int64_t nrows, double *y, double *a,
                int32_t nthreads) {
    if (check_args(type, data, scales, m, k) || !x || !y || !a || n < 1 || nrows < 1) return -1;
    if (!rows && nrows != m) return -1;
    if (rows)
        for (int64_t i = 0; i < nrows; i++)
            if (rows[i] < 0 || rows[i] >= m) return -1;

    /* x decoded once to fp64 (exact). */
    double *xd = (double *)malloc(sizeof(double) * n * k);
    if (!xd) return -1;
    for (int64_t i = 0; i < n * k; i++) xd[i] = oracle_fp16(x[i]);

    int err = 0;
#ifdef _OPENMP
    /* nthreads applies to this call only (0: the OpenMP default). */
    const int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
    g_last_threads = nth;
#else
    const int nth = 1;
    g_last_threads = 1;
#endif
    (void)nth;
#pragma omp parallel num_threads(nth)
    {
        double *w = (double *)malloc(sizeof(double) * k);
        if (!w) {
#pragma omp atomic write
            err = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = 0; i < nrows; i++) {
                int64_t r = rows ? rows[i] : i;
                dequant_row(type, data, scales, k, r, w);
                for (int64_t kk = 0; kk < k; kk++) w[kk] = (float)w[kk];   /* the fp32 weight */
                for (int64_t t = 0; t < n; t++) {
                    const double *xt = xd + t * k;
                    double acc = 0.0, acc_abs = 0.0;
                    for (int64_t kk = 0; kk < k; kk++) {
                        acc += w[kk] * xt[kk];
                        acc_abs += fabs(w[kk]) * fabs(xt[kk]);
                    }
                    y[t * nrows + i] = acc;
                    a[t * nrows + i] = acc_abs;
                }
            }
            free(w);
        }
    }
    free(xd);
    return err ? -1 : 0;
}

int32_t oracle_last_threads(void) { return g_last_threads; }

/* silu(g) = g / (1 + exp(-g)); out = silu(g) * u (kernel notes, SwiGLU section). */
void oracle_swiglu(const double *g, const double *u, int64_t len, double *out) {
    for (int64_t i = 0; i < len; i++) out[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}
