// Prefill-chunk GEMM on the matrix cores (gfx950): Y[n][m] = X[n][k] . W^T for
// n of any size, W quantized (Q4_K / Q5_K / Q6_K / NVFP4).
//
// Reference: reflex-llm Performance page, Path E / E5 -- a tensor-core K-quant
// prefill GEMM whose per-(row, sub-block) scales are decoded once and shared, and
// whose dequantized weight tile is shared by every wave of the block (E5).  Here
// a workgroup of four waves owns a BM x BN tile of Y (tokens x weight rows) and
// walks K in 128-wide steps through LDS: X[BM][128] as stored (fp16) and the
// dequantized W[BN][128]; each wave runs v_mfma_f32_16x16x32_f16 over its
// (BM/2) x (BN/2) sub-tile with fp32 accumulation.
//
// The W tile is fp16: each weight scaled by a power of two 2^(15-U) of its row, then
// rounded once to nearest even.  U bounds the magnitudes of the row's weights (|w| <
// 2^U; the largest of its superblocks' bounds, read from their d / dmin, or from
// FP8's block scales, before the K loop), so the scaled weight never overflows fp16,
// and a weight no smaller than 2^(U-29) is an fp16 normal (|error| <= 2^-11 |w|); an
// exactly zero weight stays zero.  The row's sums are scaled back (exactly) when
// stored.  NVFP4 weights are exact in fp16 and need no scale.
//
// With two LDS tile pairs (the 128x64 and 64x64 tiles) the steps are pipelined
// with one barrier each: while step s's MFMAs drain, step s+1's X (loaded into
// registers during step s-1) is written and its weights dequantized into the
// other pair, and step s+2's loads are issued; each wave reads the next 32-wide
// slice's fragments while the current slice's MFMAs run.  The 128x128 tile (and
// 64x64 in grids of more than 512 workgroups) uses one pair and two barriers per
// step, its next step's loads in flight during the MFMAs.  Loads past the last token or weight row are clamped to the
// last one (every address stays in bounds, no branches in the loop); those rows of
// the tile are never stored.  No row-invariance contract (TandemLLM Kernels page,
// "Prefill kernels"): the result is deterministic, but not the decode kernel's bits.
#include "qg_loads.hpp"
#include "qg_prefill.h"

namespace qg {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int KT = 128;   // K per step: half a superblock

// LDS tiles hold rows of KT halves, 16 chunks of 16 bytes; chunk c of row r sits at
// chunk c ^ (r & 15), so the 16 lanes of a fragment read (16 rows, one chunk each)
// hit 16 different 16-byte bank groups with no padding.
__device__ __forceinline__ int swz(int row, int c) { return row * 16 + (c ^ (row & 15)); }

// Pack two fp32 into an fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return as_u32((h2){(_Float16)lo, (_Float16)hi});
}

// One dequant task = the 64 weights of chunk c of one superblock (the probe's
// loads and unpacking are reused): step kt covers
// half s = kt & 1 of superblock kt >> 1, and its two tasks per weight row are
// chunks c = 2s + hf (hf = 0, 1).
template <int T>
__device__ __forceinline__ typename Loader<T>::Raw p_load(const PrefillArgs &A, int64_t r, int kt, int hf) {
    const int b = kt >> 1, c = 2 * (kt & 1) + hf;
    return Loader<T>::load(A.data, A.scales, A.row_bytes, r, b, c, A.tiled);
}

// Write the task's 64 weights into row `row` of the LDS weight tile (fp16, the exact
// weight times 2^(15-u) rounded once; u = the row's bound, p_row_exp), at their K
// offsets within the step (in 16-byte chunks, swizzled).
template <int T>
__device__ __forceinline__ void p_store(const typename Loader<T>::Raw &R, int kt, int hf, uint4 *tile, int row,
                                        int u) {
    const int c = 2 * (kt & 1) + hf;
    if (T == T_Q4_K || T == T_Q5_K) {
        // chunk c: sub-block 2c at step offsets 64hf + 0..31, 2c+1 at 64hf + 32..63.
        // Byte-paired quant dwords give positions (l, l+1) and (l+2, l+3) in the 16-bit
        // halves, each quant an fp16 subnormal (kq_scaled), one mixed fma per weight.
        const RawKq &Q = reinterpret_cast<const RawKq &>(R);
        const KqScaled cf = kq_scaled(Q.hdr, kq_lane_consts(c), u);
        const uint32_t qw[8] = {Q.q0.x, Q.q0.y, Q.q0.z, Q.q0.w, Q.q1.x, Q.q1.y, Q.q1.z, Q.q1.w};
        const uint32_t hw[8] = {Q.h0.x, Q.h0.y, Q.h0.z, Q.h0.w, Q.h1.x, Q.h1.y, Q.h1.z, Q.h1.w};
        uint32_t lo[16], hi[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t p = pair_bytes(qw[i], qw[i], kSelAligned), p8 = p >> 8;
            uint32_t l01 = p & 0x000F000Fu, l23 = p8 & 0x000F000Fu;
            uint32_t h01 = p & 0x00F000F0u, h23 = p8 & 0x00F000F0u;
            if (T == T_Q5_K) q5_fifth(pair_bytes(hw[i], hw[i], kSelAligned) >> (2 * c), l01, l23, h01, h23);
            lo[2 * i] = mix2(l01, cf.a0, cf.b0);
            lo[2 * i + 1] = mix2(l23, cf.a0, cf.b0);
            hi[2 * i] = mix2(h01, cf.a1, cf.b1);
            hi[2 * i + 1] = mix2(h23, cf.a1, cf.b1);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            tile[swz(row, 8 * hf + q)] = make_uint4(lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3]);
            tile[swz(row, 8 * hf + 4 + q)] = make_uint4(hi[4 * q], hi[4 * q + 1], hi[4 * q + 2], hi[4 * q + 3]);
        }
    } else if (T == T_Q6_K) {
        // half s of the superblock: group g at step offsets 32g + 16hf + 0..15
        const RawQ6 &Q = reinterpret_cast<const RawQ6 &>(R);
        const uint32_t sel = Q.mis ? kSelMis : kSelAligned;
        const uint32_t av[5] = {Q.a.x, Q.a.y, Q.a.z, Q.a.w, Q.a4};
        const uint32_t bv[5] = {Q.b.x, Q.b.y, Q.b.z, Q.b.w, Q.b4};
        const uint32_t hv[5] = {Q.h.x, Q.h.y, Q.h.z, Q.h.w, Q.h4};
        const uint32_t l0 = __builtin_amdgcn_alignbyte(Q.s01.y, Q.s01.x, Q.mis);
        const uint32_t l1 = __builtin_amdgcn_alignbyte(Q.s2, Q.s01.y, Q.mis);
        float coef[4];
        q6_coefs(l0, l1, f16lo(Q.d) * pow2f(15 - u), hf, coef);   // d scaled: exact
        uint32_t out[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const Q6Oct o = q6_oct(pair_bytes(av[i + 1], av[i], sel), pair_bytes(bv[i + 1], bv[i], sel),
                                   pair_bytes(hv[i + 1], hv[i], sel));
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float nb = (g < 2 ? -1056.0f : -384.0f) * coef[g];   // exact: coef has <= 18 bits
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    out[g][2 * i + e] = pack_h2(__builtin_fmaf(coef[g], f16lo(o.v[g][e]), nb),
                                                __builtin_fmaf(coef[g], f16hi(o.v[g][e]), nb));
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            tile[swz(row, 4 * g + 2 * hf)] = make_uint4(out[g][0], out[g][1], out[g][2], out[g][3]);
            tile[swz(row, 4 * g + 2 * hf + 1)] = make_uint4(out[g][4], out[g][5], out[g][6], out[g][7]);
        }
    } else if (T == T_FP8) {
        // FP8 chunk c: 64 codes at step offsets 64hf + 0..63, all in one 128-wide scale
        // block.  s * 2^(15-u) is exact in fp32 and code * (s * 2^(15-u)) has at most
        // 4 + 8 significant bits: rounded once to fp16.
        const RawF8 &Q = reinterpret_cast<const RawF8 &>(R);
        const float sc = bf16_lo(Q.sc) * pow2f(15 - u);
        const uint32_t qw[16] = {Q.q0.x, Q.q0.y, Q.q0.z, Q.q0.w, Q.q1.x, Q.q1.y, Q.q1.z, Q.q1.w,
                                 Q.q2.x, Q.q2.y, Q.q2.z, Q.q2.w, Q.q3.x, Q.q3.y, Q.q3.z, Q.q3.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t a = qw[2 * i], b = qw[2 * i + 1];
            tile[swz(row, 8 * hf + i)] = make_uint4(pack_h2(e4m3_at(a, 0) * sc, e4m3_at(a, 1) * sc), pack_h2(e4m3_at(a, 2) * sc, e4m3_at(a, 3) * sc),
                              pack_h2(e4m3_at(b, 0) * sc, e4m3_at(b, 1) * sc), pack_h2(e4m3_at(b, 2) * sc, e4m3_at(b, 3) * sc));
        }
    } else {
        // NVFP4 chunk c: 64 codes at step offsets 64hf + 0..63, four scales (exact, U = 15)
        const RawF4 &Q = reinterpret_cast<const RawF4 &>(R);
        const uint32_t qw[8] = {Q.q0.x, Q.q0.y, Q.q0.z, Q.q0.w, Q.q1.x, Q.q1.y, Q.q1.z, Q.q1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 sh = (_Float16)e4m3_at(Q.sc, i >> 1);   // e4m3 values are exact in fp16
            uint32_t v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = as_u32(as_h2(fp4_pair(qw[i], j)) * (h2){sh, sh});   // exact
            tile[swz(row, 8 * hf + i)] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
}

// Whether the tile's weights are scaled (every type but NVFP4).
template <int T>
constexpr bool p_scaled() { return T != T_NVFP4; }

// U of weight row r: |w| < 2^U for every weight of the row.  K-quants: the largest
// superblock bound (kq_exp_bound, q6_exp_bound); FP8: |code| <= 448 < 2^9 and a bf16
// scale with exponent field Es is below 2^(Es-126), so |w| < 2^(Es-117), clamped at
// -110 (the tiniest scales) so that 2^(15-U) stays an fp32 normal.  Reads only the
// d / dmin / scale fields, which the K loop reads again from cache.
template <int T>
__device__ __forceinline__ int p_row_exp(const PrefillArgs &A, int64_t r) {
    int u = -1000;
    const int nb = A.k / 256;
    if constexpr (T == T_Q4_K || T == T_Q5_K || T == T_Q6_K) {
        const int S = T == T_Q4_K ? 144 : (T == T_Q5_K ? 176 : 210);
#pragma unroll 8
        for (int b = 0; b < nb; ++b) {
            // d (Q6_K) or d | dmin << 16 (Q4_K, Q5_K) of row r's superblock b
            const uint8_t *f = A.tiled ? tile_chunk(A.data, nb, S, r, b) + (T == T_Q6_K ? 3328 + 2 * (r & 15) : 16 * (r & 15))
                                       : kq_block(A.data, A.row_bytes, S, r, b) + (T == T_Q6_K ? 208 : 0);
            if constexpr (T == T_Q6_K) u = max(u, q6_exp_bound(*reinterpret_cast<const uint16_t *>(f)));
            else u = max(u, kq_exp_bound(*reinterpret_cast<const uint32_t *>(f)));
        }
    } else if constexpr (T == T_FP8) {
        const uint16_t *srow = reinterpret_cast<const uint16_t *>(A.scales + (r >> 7) * (A.row_bytes / 64));
#pragma unroll 8
        for (int b = 0; b < 2 * nb; ++b) u = max(u, max((int)((srow[b] >> 7) & 0xFFu) - 117, -110));
    } else {
        u = 15;
    }
    return u;
}

// DB: double-buffered tiles, one barrier per step (see the header); otherwise one
// tile pair and two barriers per step: write step s's X and weights, barrier,
// issue step s+1's loads, MFMAs, barrier.  The 128x128 tile keeps the single buffer:
// with two, its registers no longer fit and the accumulators are shuffled between
// register files every step (measured 25 % slower); the smaller tiles gain ~10 %.
template <int T, int BM, int BN, bool DB>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs A) {
    constexpr int TM = BM / 32, TN = BN / 32;   // 16x16 MFMA tiles per wave (2 x 2 waves)
    constexpr int XC = BM * 16, WC = BN * 16;   // 16-byte chunks per X / W stage
    constexpr int XL = XC / 256;                // 16-byte X loads per thread per step
    extern __shared__ uint4 lds[];              // X stage(s), W stage(s), then the rows' U per W stage
    uint4 *const xst = lds;
    uint4 *const wst = lds + (DB ? 2 : 1) * XC;
    int *const su = reinterpret_cast<int *>(wst + (DB ? 2 : 1) * WC);   // [BN]: the rows' U

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // One-dimensional grid, row tiles fastest: (row tile, token tile) of this block.
    const int64_t rtiles = (A.m + BN - 1) / BN;
    const int64_t m0 = (int64_t)blockIdx.x / rtiles * BM;   // first token
    const int64_t n0 = (int64_t)blockIdx.x % rtiles * BN;   // first weight row
    const int nk = A.k / KT;                       // even: k is a multiple of 256
    const int last = nk - 1;

    // Dequant task of this thread: row drow, half dhf of the step's 128 weights
    // (BN rows x 2 halves; threads beyond 2 BN idle, whole waves).  Rows past m
    // read row m-1.
    const bool dq = tid < 2 * BN;
    const int drow = tid >> 1, dhf = tid & 1;
    const int64_t wr = n0 + drow < A.m ? n0 + drow : A.m - 1;

    // X: unit v of this thread is chunk c = tid % 16 of row tid / 16 + 16 v; tokens
    // past n read token n-1.
    const int64_t kv = A.k / 8;   // 16-byte units per X row
    const u32x4 *xt = reinterpret_cast<const u32x4 *>(A.x) + m0 * kv + (tid & 15);
    int xo[XL];
#pragma unroll
    for (int v = 0; v < XL; ++v) {
        const int64_t t = m0 + (tid >> 4) + 16 * v;
        xo[v] = (int)(((t < A.n ? t : A.n - 1) - m0) * kv);
    }
    auto load_x = [&](u32x4 (&xv)[XL], int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < XL; ++v) xv[v] = xt[xo[v] + kt * (KT / 8)];
    };
    auto store_x = [&](const u32x4 (&xv)[XL], int stage) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < XL; ++v)
            *reinterpret_cast<u32x4 *>(xst + stage * XC + swz((tid >> 4) + 16 * v, tid & 15)) = xv[v];
    };

    f4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f4){0.f, 0.f, 0.f, 0.f};

    const int arow = wm * (BM / 2) + (lane & 15), brow = wn * (BN / 2) + (lane & 15);
    // The dequant thread's row exponent; the MFMA lanes read their rows' from LDS at
    // the end (su is written before the loop's first barrier).
    const int urow = dq ? p_row_exp<T>(A, wr) : 15;
    if (dq && dhf == 0) su[drow] = urow;
    if constexpr (!DB) {
        typename Loader<T>::Raw raw;
        u32x4 xv[XL];
        if (dq) raw = p_load<T>(A, wr, 0, dhf);
        load_x(xv, 0);
        for (int s = 0; s < nk; ++s) {
            __syncthreads();   // the previous step's readers are done
            store_x(xv, 0);
            if (dq) p_store<T>(raw, s, dhf, wst, drow, urow);
            __syncthreads();
            if (s + 1 < nk) {   // in flight during this step's MFMAs
                load_x(xv, s + 1);
                if (dq) raw = p_load<T>(A, wr, s + 1, dhf);
            }
#pragma unroll
            for (int ks = 0; ks < KT / 32; ++ks) {
                const int c = 4 * ks + (lane >> 4);
                h8 af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const h8 *>(xst + swz(arow + 16 * i, c));
#pragma unroll
                for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const h8 *>(wst + swz(brow + 16 * j, c));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        }
    } else {
        // One register slot per stream: loaded during step s, written to LDS during
        // step s+1.  Step indexes past the end are clamped (redundant, in-bounds loads).
        typename Loader<T>::Raw raw;
        u32x4 xv[XL];
        if (dq) raw = p_load<T>(A, wr, 0, dhf);
        load_x(xv, 0);
        store_x(xv, 0);
        if (dq) {
            p_store<T>(raw, 0, dhf, wst, drow, urow);
            raw = p_load<T>(A, wr, 1, dhf);
        }
        load_x(xv, 1);

        for (int s = 0; s < nk; ++s) {
            // Every wave's part of step s's tiles is in LDS, and every wave is done
            // with step s-1's tiles (rewritten below with step s+1).
            __syncthreads();
            const int p = s & 1;
            const uint4 *xs = xst + p * XC;
            const uint4 *ws = wst + p * WC;
            h8 af[2][TM], bf[2][TN];
    #pragma unroll
            for (int i = 0; i < TM; ++i) af[0][i] = *reinterpret_cast<const h8 *>(xs + swz(arow + 16 * i, lane >> 4));
    #pragma unroll
            for (int j = 0; j < TN; ++j) bf[0][j] = *reinterpret_cast<const h8 *>(ws + swz(brow + 16 * j, lane >> 4));
    #pragma unroll
            for (int ks = 0; ks < KT / 32; ++ks) {
                const int cur = ks & 1;
                if (ks + 1 < KT / 32) {
                    const int c = 4 * (ks + 1) + (lane >> 4);
    #pragma unroll
                    for (int i = 0; i < TM; ++i) af[cur ^ 1][i] = *reinterpret_cast<const h8 *>(xs + swz(arow + 16 * i, c));
    #pragma unroll
                    for (int j = 0; j < TN; ++j) bf[cur ^ 1][j] = *reinterpret_cast<const h8 *>(ws + swz(brow + 16 * j, c));
                }
    #pragma unroll
                for (int i = 0; i < TM; ++i)
    #pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[cur][i], bf[cur][j], acc[i][j], 0, 0, 0);
            }
            // step s+1 into the other tiles (last read in step s-1) while the last
            // MFMAs drain, then load step s+2
            const int s1 = s + 1 < last ? s + 1 : last, s2 = s + 2 < last ? s + 2 : last;
            store_x(xv, p ^ 1);
            load_x(xv, s2);
            if (dq) {
                p_store<T>(raw, s1, dhf, wst + (p ^ 1) * WC, drow, urow);
                raw = p_load<T>(A, wr, s2, dhf);
            }
        }
    }
    // D tile (i, j): lane holds tokens 4*(lane/16)+e, weight row lane%16.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t r = n0 + wn * (BN / 2) + 16 * j + (lane & 15);
            const float back = p_scaled<T>() ? pow2f(su[wn * (BN / 2) + 16 * j + (lane & 15)] - 15) : 1.0f;   // exact
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = m0 + wm * (BM / 2) + 16 * i + 4 * (lane >> 4) + e;
                if (t < A.n && r < A.m) A.y[t * A.m + r] = acc[i][j][e] * back;
            }
        }
}

template <int T, int BM, int BN, bool DB>
static hipError_t launch_tile(const PrefillArgs &A, hipStream_t st) {
    const int64_t blocks = (A.m + BN - 1) / BN * ((A.n + BM - 1) / BM);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const size_t lds = (size_t)(BM + BN) * 256 * (DB ? 2 : 1) + (size_t)BN * 4;
    const void *fn = (const void *)prefill_kernel<T, BM, BN, DB>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((prefill_kernel<T, BM, BN, DB>), grid, dim3(256), lds, st, A);
    return hipGetLastError();
}

template <int T>
static hipError_t launch_t(const PrefillArgs &A, int bm, int bn, hipStream_t st) {
    if (bm == 128 && bn == 128) return launch_tile<T, 128, 128, false>(A, st);
    if (bm == 128) return launch_tile<T, 128, 64, true>(A, st);
    // Two 64x64 tile pairs (64 KB) leave room for two workgroups per CU; past 512
    // workgroups the single pair (32 KB) keeps them all resident at once.
    if ((A.m + 63) / 64 * ((A.n + 63) / 64) > 512) return launch_tile<T, 64, 64, false>(A, st);
    return launch_tile<T, 64, 64, true>(A, st);
}

hipError_t launch_prefill(const PrefillArgs &A, int bm, int bn, hipStream_t st) {
    switch (A.type) {
    case T_Q4_K: return launch_t<T_Q4_K>(A, bm, bn, st);
    case T_Q5_K: return launch_t<T_Q5_K>(A, bm, bn, st);
    case T_Q6_K: return launch_t<T_Q6_K>(A, bm, bn, st);
    case T_FP8: return launch_t<T_FP8>(A, bm, bn, st);
    default: return launch_t<T_NVFP4>(A, bm, bn, st);
    }
}

}  // namespace qg
