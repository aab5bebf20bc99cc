/*
 * qgemm.h -- C ABI of libqgemm.so, the fused dequantize-in-registers product
 *
 *     y[n x m] = x[n x k] . W^T        (W quantized, x fp16, y fp32)
 *
 * for GGML K-quant weights (Q4_K, Q5_K, Q6_K) and NVFP4 W4A16 weights, on an
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (page title, then section):
 *  [KN]  reflex-llm kernel notes (docs/kernels.md): the K-quant GEMV, the
 *        uint32 weight-load variant with its residual-add / pair / triple
 *        kernels, and the batched multi-token GEMM.
 *  [PF]  reflex-llm Performance page: Path C (Q4_K uint32 decode loads, the
 *        210-byte Q6_K block), Path E / E5 (tensor-core Q4_K prefill GEMM).
 *  [TK]  TandemLLM Kernels page: "Row invariance", "Verify twins",
 *        "NVFP4 matrix products", "Head, norms, attention".
 *
 * Conventions shared by every entry point
 *  - All buffer pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, frees nothing and keeps no mutable state; calls may be
 *    made from several host threads at once.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work
 *    and return; results are ready when the stream reaches that point.
 *  - x is fp16, row-major [n][k], contiguous.  y and resid are fp32 row-major
 *    [n][m]: output (token t, weight row r) is y[t*m + r]  ([KN] batched GEMM,
 *    output layout).
 *  - W is stored exactly as the format defines, rows contiguous:
 *      Q4_K: 144-byte superblocks of 256 weights: fp16 d, fp16 dmin, 12 bytes
 *            of packed 6-bit sub-block scales/mins, 128 bytes of 4-bit quants;
 *      Q5_K: 176-byte superblocks: as Q4_K plus 32 bytes of fifth quant bits
 *            (placed before the 128 quant bytes);
 *      Q6_K: 210-byte superblocks: 128 bytes of low 4 bits, 64 bytes of high
 *            2 bits, 16 int8 sub-block scales, fp16 d;
 *      NVFP4: `data` = e2m1 codes [m][k/2] (element k in byte k/2, low nibble
 *            for even k); `scales` = e4m3 (OCP E4M3FN) [m][k/16], one per 16
 *            consecutive weights of a row.
 *    Weight value: Q4_K/Q5_K  d*sc[j]*q - dmin*min[j]  ([PF] Path E);
 *                  Q6_K       d*sc[j]*(q - 32);
 *                  NVFP4      e2m1(code) * e4m3(scale)  ([TK] NVFP4).
 *    Row r of a K-quant weight starts at data + r * qg_row_bytes(type, k)
 *    (QG_LAYOUT_ROWS, the layout the superblocks are stored in), or, in the
 *    16-row tiled layout (QG_LAYOUT_TILES, made by qg_pack_tiles), superblock b of
 *    the 16 rows of tile r/16 is one chunk of 16*S bytes at data + (r/16 * (k/256)
 *    + b) * 16 * S, S the superblock size, with the bytes of those 16 superblocks
 *    arranged so that every 16-byte load of the product kernel reads a run shared
 *    with its neighbour lanes (the arrangement of each type is documented with
 *    the loads in qg_loads.hpp).  The values are the same; so are the bits of
 *    every product.
 *  - k must be a multiple of 256 for every type (one superblock; for NVFP4 one
 *    block of 16 scales).  m >= 1.
 *  - Alignment: data, scales and x 16-byte aligned; y and resid 4-byte aligned.
 *  - Errors: every argument is checked on the host BEFORE anything is enqueued;
 *    on error nothing is launched and a negative QG_ERR_* code is returned, with
 *    a description in qg_last_error() (thread-local).  There is no fallback
 *    kernel.  Weight contents are not validated (NaN codes propagate).
 *  - Aliasing: resid may equal y (in-place residual add); any other overlap
 *    between an output and another buffer is undefined.
 *  - Determinism and row invariance ([TK] Row invariance, Verify twins): the
 *    arithmetic of a row -- its operands, its K phases and the order their sums
 *    are added in -- depends only on (type, m, k), never on n or on the other
 *    rows; the launch shape (waves per workgroup, phases per wave, how x is
 *    staged) may follow n without touching it.  For 1 <= n <= 32 the
 *    qgemv_* / qgemm_rows / fused calls therefore give bit-identical results
 *    for a given row whether it is called alone (n = 1) or as one of n rows,
 *    each output of a pair/triple equals the corresponding single call bit for
 *    bit, and qgemv_add equals fl32(resid + qgemm_rows(...)).  Repeated calls
 *    return identical bits.  qgemm_prefill is deterministic but carries no such
 *    twin contract ([TK] "Prefill kernels": chunk kernels share work across rows).
 *  - Accuracy: a Q4_K / Q5_K weight enters the product exactly, split as
 *    d*sc*(q - c) + r with c the integer nearest to dmin*m/(d*sc) (an exact fp16
 *    operand times d, and a per-sub-block fp32 remainder r times the sub-block's
 *    sum of x), both parts bounded by the weight; a Q6_K weight enters as the fp16
 *    operand (q - 32)*sc*2^-16 times d*2^16, exact for |sc| <= 64 and otherwise
 *    rounded once (relative error <= 2^-11); FP8 and NVFP4 weights enter exactly
 *    (the e4m3 code, or e2m1 times its e4m3 scale, is exact in fp16, and the
 *    block scales are applied in fp32).
 *    With fp32 accumulation |y - y_exact| stays within 2e-3 * sum_k |w||x| also
 *    where the two terms of a Q4_K / Q5_K weight cancel, and an output whose
 *    weights are all zero is exactly zero (exactly resid for qgemv_add).
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tensor type codes.  12 and 14 are the GGML type numbers of Q4_K and Q6_K that
 * [PF] Path C's typed kernels are instantiated with (<12>, <12,12>, <12,12,14>);
 * 13 (Q5_K) sits between them; NVFP4 and block-scaled FP8 have no GGML number and
 * take 1001 and 1002. */
typedef enum {
    QG_Q4_K = 12,
    QG_Q5_K = 13,
    QG_Q6_K = 14,
    QG_NVFP4 = 1001,
    QG_FP8 = 1002   /* [TK] "FP8 matrix products": e4m3 codes, one bf16 scale per 128x128 block */
} qg_type;

/* Status codes. */
#define QG_OK            0
#define QG_ERR_NULL     -1   /* a required pointer is NULL                        */
#define QG_ERR_SHAPE    -2   /* m < 1, k not a multiple of 256, k mismatch, n < 1 */
#define QG_ERR_ROWS     -3   /* n outside 1..QG_MAX_ROWS for a row-invariant call */
#define QG_ERR_TYPE     -4   /* unknown type, or a type the call does not take    */
#define QG_ERR_ALIGN    -5   /* a pointer violates the alignment rules            */
#define QG_ERR_LAUNCH   -6   /* the HIP runtime refused the launch                */

#define QG_MAX_ROWS 32       /* largest n of the row-invariant calls ([KN] GEMM_MAX_BATCH) */

#define QG_LAYOUT_ROWS  0    /* rows one after another, as stored               */
#define QG_LAYOUT_TILES 1    /* K-quants in 16-row tiles (see qg_pack_tiles)     */

/* A quantized weight matrix (m rows of k weights).  `scales` is used by NVFP4 and
 * FP8 and must be non-NULL (16-byte aligned) for them; it is ignored for the
 * K-quants.  FP8: data = e4m3 codes [m][k] (OCP E4M3FN, one byte per weight), scales
 * = bf16 [ceil(m/128)][k/128] row-major, weight (r, c) = code * scale[r/128][c/128]. */
typedef struct qg_weight {
    int32_t type;        /* a qg_type                                   */
    int32_t layout;      /* QG_LAYOUT_ROWS (0) or QG_LAYOUT_TILES (1)    */
    const void *data;    /* superblocks, or NVFP4 / FP8 codes           */
    const void *scales;  /* NVFP4 e4m3 [m][k/16]; FP8 bf16 [m/128][k/128] */
    int64_t m;           /* rows (output features)                      */
    int64_t k;           /* columns (reduction length)                  */
} qg_weight;

/* Bytes of one stored weight row (NVFP4 and FP8: of the codes only); -1 if the
 * type is unknown or k is not a multiple of 256. */
int64_t qg_row_bytes(int32_t type, int64_t k);

/*
 * The 16-row tiled layout of a K-quant matrix (an MI355X-side layout choice, not a
 * format of the pages): qg_tiles_bytes gives the size of the tiled copy of w,
 * 16 * ceil(m/16) * qg_row_bytes (the rows past m in the last tile repeat row
 * m-1), or a negative error (QG_ERR_TYPE for NVFP4/FP8).  qg_pack_tiles writes that
 * copy of w (which must be in QG_LAYOUT_ROWS) to dst (device, 16-byte aligned, owned
 * by the caller; must not overlap w->data); describe it with layout =
 * QG_LAYOUT_TILES and the same type, m and k.  Every call accepts both layouts
 * (the single-token qgemv_q4k/q5k/q6k take the row layout only).
 */
int64_t qg_tiles_bytes(const qg_weight *w);
int qg_pack_tiles(const qg_weight *w, void *dst, void *stream);

/* Static text for a status code. */
const char *qg_status_str(int status);

/* Description of the last error raised on the calling thread ("" if none). */
const char *qg_last_error(void);

/*
 * Single-token GEMV, one call per weight type ([KN] K-quant GEMV: y[M] = W[MxK] x[K];
 * the dispatcher there selects the kernel by GGML tensor type).
 *   w: m rows of the named type; x: fp16 [k]; y: fp32 [m].
 * Bit-identical to qgemm_rows with n = 1 on the same weight ([KN]: N = 1 routes to
 * the GEMV so the decode path is bit-identical).
 */
int qgemv_q4k(const void *w, const void *x, float *y, int64_t m, int64_t k, void *stream);
int qgemv_q5k(const void *w, const void *x, float *y, int64_t m, int64_t k, void *stream);
int qgemv_q6k(const void *w, const void *x, float *y, int64_t m, int64_t k, void *stream);

/* Block-scaled FP8 W8A16 GEMV ([TK] FP8 matrix products: the checkpoint's e4m3
 * codes with one bf16 scale per 128 x 128 block, read as stored): codes [m][k],
 * scales bf16 [ceil(m/128)][k/128], x fp16 [k], y fp32 [m].  k a multiple of 256.
 * Each 128-wide block's sum of code*x is formed on the matrix cores (codes exact in
 * fp16) and scaled in fp32; row-invariant like every other type. */
int qgemv_fp8(const void *codes, const void *scales, const void *x, float *y, int64_t m, int64_t k,
              void *stream);

/* NVFP4 W4A16 GEMV ([TK] NVFP4 matrix products): codes [m][k/2], scales e4m3
 * [m][k/16], x fp16 [k], y fp32 [m]. */
int qgemv_nvfp4(const void *codes, const void *scales, const void *x, float *y,
                int64_t m, int64_t k, void *stream);

/*
 * Row-invariant multi-token product, 1 <= n <= 32 ([KN] batched GEMM: weights are
 * streamed once for n tokens; [TK] Verify twins: the n-row call equals n one-row
 * calls bit for bit).  x fp16 [n][k], y fp32 [n][m].
 */
int qgemm_rows(const qg_weight *w, const void *x, float *y, int32_t n, void *stream);

/*
 * Residual-fused product ([KN] gemv_quant_add: the Wo projection with the residual
 * add folded in):  y[t][r] = fl32(resid[t][r] + (x W^T)[t][r]),  1 <= n <= 32.
 * resid may be the same buffer as y.
 */
int qgemv_add(const qg_weight *w, const void *x, const float *resid, float *y,
              int32_t n, void *stream);

/*
 * Two products sharing x in one launch ([KN] gemv_quant_pair: gate and up).
 * w0->k must equal w1->k; types may differ.  y0 [n][w0->m], y1 [n][w1->m].
 */
int qgemv_pair(const qg_weight *w0, const qg_weight *w1, const void *x,
               float *y0, float *y1, int32_t n, void *stream);

/*
 * Three products sharing x in one launch ([KN] gemv_quant_triple: Q, K, V with
 * the Q4_K/Q4_K/Q6_K mix of Qwen3-4B Q4_K_M).  All k equal; types may differ.
 */
int qgemv_triple(const qg_weight *w0, const qg_weight *w1, const qg_weight *w2,
                 const void *x, float *y0, float *y1, float *y2, int32_t n, void *stream);

/*
 * Gate/up pair with the SwiGLU activation fused into its epilogue ([KN] SwiGLU:
 * out = silu(gate) * up, silu(g) = g / (1 + exp(-g))):
 *   h[t][r] = silu((x Wg^T)[t][r]) * (x Wu^T)[t][r],  1 <= n <= 32.
 * wg and wu must have the same m and k.  h fp32 [n][m].  The two products are
 * the bits of qgemv_pair; the activation adds one fp32 evaluation.
 */
int qgemv_pair_swiglu(const qg_weight *wg, const qg_weight *wu, const void *x,
                      float *h, int32_t n, void *stream);

/*
 * Prefill-chunk GEMM on the matrix cores ([PF] Path E / E5: tensor-core K-quant
 * prefill GEMM with scales decoded once per (row, sub-block) and one dequantized
 * weight tile shared by all waves of a block): Y[n][m] = X[n][k] W^T for any
 * n >= 1 and every weight type.  Each wave decodes the weights of its 16 rows
 * once per 64 tokens into MFMA operands in registers (the operands and per-
 * superblock arithmetic of the 1..32-token calls, described under Accuracy) and
 * multiplies with v_mfma_f32_16x16x32_f16, fp32 accumulation.  x fp16 [n][k],
 * y fp32 [n][m].  n up to 2^30; QG_ERR_SHAPE if the call would need more than
 * 2^31 - 1 blocks of Y (64 x 64 each).  Deterministic; no row-invariance
 * contract ([TK] "Prefill kernels": chunk kernels share work across rows and are
 * checked by agreement).
 */
int qgemm_prefill(const qg_weight *w, const void *x, float *y, int64_t n, void *stream);

/*
 * Decoder probe: out[r][k] = the fp32 weight value of row r, column k, for every
 * element (the device decoders the products use).  out fp32 [m][k].
 */
int qdequant(const qg_weight *w, float *out, void *stream);

/*
 * Read-stream probe, a measuring stick and not part of any product: reads the
 * nreg (1..3) device regions ptrs[i] of bytes[i] bytes each once, with 16-byte
 * vector loads and no arithmetic on the data, and XORs every 32-bit word of them
 * into out, a device array of 2048 uint32 (128-byte aligned, updated in place and
 * not cleared): the XOR of all 2048 words changes by the XOR of all words read.
 * Timing it over the bytes a weight product streams gives the plain HBM read rate
 * the product is compared with.  ptrs and bytes are host arrays; every region is
 * 16-byte aligned and bytes[i] is a positive multiple of 16.  Errors: QG_ERR_NULL,
 * QG_ERR_SHAPE, QG_ERR_ALIGN, QG_ERR_LAUNCH; nothing is launched on error.
 */
int qg_stream_read(const void *const *ptrs, const int64_t *bytes, int32_t nreg, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMM_H */
