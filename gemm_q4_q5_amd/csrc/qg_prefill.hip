// Prefill-chunk GEMM on the matrix cores (gfx950): Y[n][m] = X[n][k] . W^T for
// n of any size, W quantized (Q4_K / Q5_K / Q6_K / NVFP4).
//
// Reference: reflex-llm Performance page, Path E / E5 -- a tensor-core K-quant
// prefill GEMM whose per-(row, sub-block) scales are decoded once and shared, and
// whose dequantized weight tile is shared by every wave of the block (E5).  Here
// a workgroup of four waves owns a BM x BN tile of Y (tokens x weight rows) and
// walks K in 128-wide steps: it stages X[BM][128] and the dequantized W[BN][128]
// (fp16: the exact weight rounded once, to nearest even; |error| <= 2^-11 |w|) in LDS,
// then each wave runs v_mfma_f32_16x16x32_f16 over its (BM/2) x (BN/2) sub-tile
// with fp32 accumulation.  The next step's global loads are issued before the
// current step's MFMAs.  No row-invariance contract (TandemLLM Kernels page,
// "Prefill kernels"): the result is deterministic, but not the decode kernel's bits.
#include "qg_loads.hpp"
#include "qg_prefill.h"

namespace qg {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int KT = 128;       // K per step: half a superblock
constexpr int KP = KT + 8;    // LDS row pitch in halves (16 bytes of padding)

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

// Write the task's 64 weights (fp16, one rounding of the exact fp32 value) into
// the LDS row of the step, at their K offsets within the step.
template <int T>
__device__ __forceinline__ void p_store(const typename Loader<T>::Raw &R, int kt, int hf, _Float16 *wrow) {
    const int c = 2 * (kt & 1) + hf;
    if (T == T_Q4_K || T == T_Q5_K) {
        // chunk c: sub-block 2c at step offsets 64hf + 0..31, 2c+1 at 64hf + 32..63
        const RawKq &Q = reinterpret_cast<const RawKq &>(R);
        const KqCoef cf = kq_coef(Q.hdr, kq_lane_consts(c));
        // w = a*q + b with the exact products a = d*sc, b = -dmin*m: q is recovered
        // exactly from the fp16 magic value (v - 1024, v - 256 = 4q).  The fma and
        // the fp16 conversion compile to one mixed-precision fma with an fp16 result
        // (v_fma_mix{lo,hi}_f16), which rounds the exact a*q + b once, straight to
        // fp16; an fp32 result rounded again to fp16 would differ where the fp32
        // value lands on an fp16 tie.
        const uint32_t qw[8] = {Q.q0.x, Q.q0.y, Q.q0.z, Q.q0.w, Q.q1.x, Q.q1.y, Q.q1.z, Q.q1.w};
        const uint32_t hw[8] = {Q.h0.x, Q.h0.y, Q.h0.z, Q.h0.w, Q.h1.x, Q.h1.y, Q.h1.z, Q.h1.w};
        const h2 m0 = {(_Float16)1024.0f, (_Float16)1024.0f}, m1 = {(_Float16)256.0f, (_Float16)256.0f};
        uint32_t lo[16], hi[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const Quad qd = T == T_Q5_K ? q5_quad(qw[i], pair_bytes(hw[i], hw[i], kSelAligned) >> (2 * c))
                                        : q4_quad(qw[i]);
            const h2 p0 = as_h2(qd.lo01) - m0, p1 = as_h2(qd.lo23) - m0;   // exact small integers
            const h2 p2 = as_h2(qd.hi01) - m1, p3 = as_h2(qd.hi23) - m1;
            lo[2 * i] = pack_h2(__builtin_fmaf(cf.a0, (float)p0.x, cf.b0), __builtin_fmaf(cf.a0, (float)p0.y, cf.b0));
            lo[2 * i + 1] = pack_h2(__builtin_fmaf(cf.a0, (float)p1.x, cf.b0), __builtin_fmaf(cf.a0, (float)p1.y, cf.b0));
            hi[2 * i] = pack_h2(__builtin_fmaf(cf.a1, (float)p2.x, cf.b1), __builtin_fmaf(cf.a1, (float)p2.y, cf.b1));
            hi[2 * i + 1] = pack_h2(__builtin_fmaf(cf.a1, (float)p3.x, cf.b1), __builtin_fmaf(cf.a1, (float)p3.y, cf.b1));
        }
        uint4 *dl = reinterpret_cast<uint4 *>(wrow + 64 * hf);
        uint4 *dh = reinterpret_cast<uint4 *>(wrow + 64 * hf + 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            dl[q] = make_uint4(lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3]);
            dh[q] = make_uint4(hi[4 * q], hi[4 * q + 1], hi[4 * q + 2], hi[4 * q + 3]);
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
        q6_coefs(l0, l1, f16lo(Q.d), hf, coef);
        uint32_t out[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const Q6Oct o = q6_oct(pair_bytes(av[i + 1], av[i], sel), pair_bytes(bv[i + 1], bv[i], sel),
                                   pair_bytes(hv[i + 1], hv[i], sel));
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float nb = (g < 2 ? -1056.0f : -384.0f) * coef[g];   // exact: coef has <= 19 bits
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    out[g][2 * i + e] = pack_h2(__builtin_fmaf(coef[g], f16lo(o.v[g][e]), nb),
                                                __builtin_fmaf(coef[g], f16hi(o.v[g][e]), nb));
            }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint4 *d = reinterpret_cast<uint4 *>(wrow + 32 * g + 16 * hf);
            d[0] = make_uint4(out[g][0], out[g][1], out[g][2], out[g][3]);
            d[1] = make_uint4(out[g][4], out[g][5], out[g][6], out[g][7]);
        }
    } else if (T == T_FP8) {
        // FP8 chunk c: 64 codes at step offsets 64hf + 0..63; code * scale is exact in
        // fp32 (4 + 8 significant bits) and rounded once to fp16.
        const RawF8 &Q = reinterpret_cast<const RawF8 &>(R);
        const float sc = bf16_lo(Q.sc);
        const uint32_t qw[16] = {Q.q0.x, Q.q0.y, Q.q0.z, Q.q0.w, Q.q1.x, Q.q1.y, Q.q1.z, Q.q1.w,
                                 Q.q2.x, Q.q2.y, Q.q2.z, Q.q2.w, Q.q3.x, Q.q3.y, Q.q3.z, Q.q3.w};
        uint4 *d = reinterpret_cast<uint4 *>(wrow + 64 * hf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t a = qw[2 * i], b = qw[2 * i + 1];
            d[i] = make_uint4(pack_h2(e4m3_at(a, 0) * sc, e4m3_at(a, 1) * sc), pack_h2(e4m3_at(a, 2) * sc, e4m3_at(a, 3) * sc),
                              pack_h2(e4m3_at(b, 0) * sc, e4m3_at(b, 1) * sc), pack_h2(e4m3_at(b, 2) * sc, e4m3_at(b, 3) * sc));
        }
    } else {
        // NVFP4 chunk c: 64 codes at step offsets 64hf + 0..63, four scales
        const RawF4 &Q = reinterpret_cast<const RawF4 &>(R);
        const uint32_t qw[8] = {Q.q0.x, Q.q0.y, Q.q0.z, Q.q0.w, Q.q1.x, Q.q1.y, Q.q1.z, Q.q1.w};
        uint4 *d = reinterpret_cast<uint4 *>(wrow + 64 * hf);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 sh = (_Float16)e4m3_at(Q.sc, i >> 1);   // e4m3 values are exact in fp16
            uint32_t v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = as_u32(as_h2(fp4_pair(qw[i], j)) * (h2){sh, sh});   // exact
            d[i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int T, int BM, int BN>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs A) {
    constexpr int TM = BM / 32, TN = BN / 32;      // 16x16 MFMA tiles per wave (2 x 2 waves)
    constexpr int XV = BM * KT / 8 / 256;          // 16-byte X loads per thread per step
    __shared__ __align__(16) _Float16 xs[BM * KP];
    __shared__ __align__(16) _Float16 ws[BN * KP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;   // first token
    const int64_t n0 = (int64_t)blockIdx.x * BN;   // first weight row
    const int nk = A.k / KT;

    // dequant task of this thread (BN rows x 2 chunks per step; threads beyond idle)
    const bool dq = tid < 2 * BN;
    const int drow = tid >> 1, dhf = tid & 1;
    const int64_t wr = n0 + drow;
    const bool wvalid = dq && wr < A.m;

    f4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f4){0.f, 0.f, 0.f, 0.f};

    const uint4 *xg = reinterpret_cast<const uint4 *>(A.x);
    uint4 xv[XV];
    typename Loader<T>::Raw raw;
    auto fetch = [&](int kt) {
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int i = tid + 256 * v;          // 16-byte unit of the X tile
            const int row = i >> 4, col = i & 15;  // 16 units per 128-wide row
            const int64_t t = m0 + row;
            xv[v] = t < A.n ? xg[(t * A.k + (int64_t)kt * KT) / 8 + col] : make_uint4(0, 0, 0, 0);
        }
        if (wvalid) raw = p_load<T>(A, wr, kt, dhf);
    };
    fetch(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();   // the previous step's readers are done
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int i = tid + 256 * v;
            *reinterpret_cast<uint4 *>(xs + (i >> 4) * KP + (i & 15) * 8) = xv[v];
        }
        if (dq) {
            _Float16 *wrow = ws + drow * KP;
            if (wvalid) {
                p_store<T>(raw, kt, dhf, wrow);
            } else {   // rows past m: zeros (NVFP4/K-quant halves each cover 64 of the 128)
                for (int q = 0; q < 8; ++q) reinterpret_cast<uint4 *>(wrow)[8 * dhf + q] = make_uint4(0, 0, 0, 0);
            }
        }
        __syncthreads();
        if (kt + 1 < nk) fetch(kt + 1);   // in flight during this step's MFMAs
#pragma unroll
        for (int ks = 0; ks < KT / 32; ++ks) {
            h8 af[TM], bf[TN];
            const int kof = ks * 32 + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const h8 *>(xs + (wm * (BM / 2) + 16 * i + (lane & 15)) * KP + kof);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = *reinterpret_cast<const h8 *>(ws + (wn * (BN / 2) + 16 * j + (lane & 15)) * KP + kof);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }
    // D tile (i, j): lane holds tokens 4*(lane/16)+e, weight row lane%16.
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t r = n0 + wn * (BN / 2) + 16 * j + (lane & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = m0 + wm * (BM / 2) + 16 * i + 4 * (lane >> 4) + e;
                if (t < A.n && r < A.m) A.y[t * A.m + r] = acc[i][j][e];
            }
        }
}

template <int T>
static hipError_t launch_t(const PrefillArgs &A, int bm, int bn, hipStream_t st) {
    const dim3 grid((unsigned)((A.m + bn - 1) / bn), (unsigned)((A.n + bm - 1) / bm));
    if (bm == 128 && bn == 128)
        hipLaunchKernelGGL((prefill_kernel<T, 128, 128>), grid, dim3(256), 0, st, A);
    else if (bm == 128)
        hipLaunchKernelGGL((prefill_kernel<T, 128, 64>), grid, dim3(256), 0, st, A);
    else
        hipLaunchKernelGGL((prefill_kernel<T, 64, 64>), grid, dim3(256), 0, st, A);
    return hipGetLastError();
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
