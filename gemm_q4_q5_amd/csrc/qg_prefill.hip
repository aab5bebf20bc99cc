// Prefill-chunk GEMM on the matrix cores (gfx950): Y[n][m] = X[n][k] . W^T for
// n of any size, W quantized (Q4_K / Q5_K / Q6_K / NVFP4 / FP8).
//
// Reference: reflex-llm Performance page, Path E / E5 -- a tensor-core K-quant
// prefill GEMM whose per-(row, sub-block) scales are decoded once and whose
// dequantized weights serve many tokens.  Here a workgroup owns a block of 16*NG
// tokens by 64*NT weight rows.  Each of its four waves owns NT row tiles (16 rows
// each) and builds their v_mfma_f32_16x16x32_f16 weight operands in its own
// registers, straight from the streamed superblocks (the same loads and unpacking
// as the 1..32-token product), so a weight is decoded once per token block and
// never passes through LDS.  The block's tokens (fp16) are staged in LDS once per
// superblock, in the operand's k-slot order, and every wave reads them from there.
// Per superblock and step a wave reads NG x fragments and issues NT*NG MFMAs.
//
// Weight operands are those of the 1..32-token product: Q4_K / Q5_K through the exact
// split (kq_split: an exact fp16 operand per weight, one MFMA chain per superblock
// scaled by d, the sub-blocks' remainders times their x sums through fp32 MFMAs), so
// no weight is rounded; Q6_K as (q - 32)*sc*2^-16 in fp16 (exact for |sc| <= 64, else
// rounded once), one chain per superblock scaled by d*2^16; NVFP4 exact.  FP8 operands
// are the weight times a power of two 2^(15-U) of its row, rounded once to fp16: U
// bounds the row's weights (read from its block scales before the K loop), so the
// scaled weight never overflows fp16 and a weight no smaller than 2^(U-29) is an fp16
// normal (|error| <= 2^-11 |w|); the row's sums are scaled back exactly when stored.
//
// Per superblock b: b+1's weights and x are loaded into registers while b is
// computed; a barrier; b+1's x is written to the (single) LDS buffer; a barrier.
// Several workgroups share a CU, so one's barriers overlap another's MFMAs.  Loads
// past the last token or weight row are clamped to the last one (every address
// stays in bounds); those rows are never stored.  No row-invariance contract
// (TandemLLM Kernels page, "Prefill kernels"): the result is deterministic, but not
// the decode kernel's bits.
#include <type_traits>

#include "qg_loads.hpp"
#include "qg_mma.hpp"
#include "qg_prefill.h"

namespace qg {

// U of weight row r (FP8; 15 for the others): |w| < 2^U for every weight of the row.  FP8: |code| <= 448 < 2^9 and a bf16
// scale with exponent field Es is below 2^(Es-126), so |w| < 2^(Es-117), clamped at
// -110 (the tiniest scales) so that 2^(15-U) stays an fp32 normal.  Reads only the
// d / dmin / scale fields, which the K loop reads again from cache.
template <int T>
__device__ __forceinline__ int p_row_exp(const PrefillArgs &A, int64_t r) {
    int u = 15;
    if constexpr (T == T_FP8) {
        const int nb = A.k / 256;
        const uint16_t *srow = reinterpret_cast<const uint16_t *>(A.scales + (r >> 7) * (A.row_bytes / 64));
        u = -1000;
#pragma unroll 8
        for (int b = 0; b < 2 * nb; ++b) u = max(u, max((int)((srow[b] >> 7) & 0xFFu) - 117, -110));
    }
    return u;
}

// Whether the weights are scaled by a power of two of their row (FP8; Q4_K and Q5_K
// use the exact split, Q6_K a per-superblock chain scaled by d, NVFP4 is exact in fp16).
template <int T>
constexpr bool p_scaled() { return T == T_FP8; }

// Per-tile coefficients of one superblock for the lane's row (u = the row's U).
struct PCoefKq {
    KqSplit k;
};
struct PCoefQ6 {
    Q6Tile k;
};
struct PCoefF8 {
    float a[2];         // block h weight = fp16(a[h] * code)
};
template <int T>
struct PCoefOf {
    typedef PCoefKq type;
};
template <>
struct PCoefOf<T_Q6_K> {
    typedef PCoefQ6 type;
};
template <>
struct PCoefOf<T_FP8> {
    typedef PCoefF8 type;
};
template <>
struct PCoefOf<T_NVFP4> {
    typedef int type;   // exact operands, nothing to scale
};

template <int T>
__device__ __forceinline__ typename PCoefOf<T>::type p_coef(const typename MRawOf<T>::type &R, const KqLane &L,
                                                            int g, int u) {
    typename PCoefOf<T>::type c;
    if constexpr (T == T_Q4_K || T == T_Q5_K) {
        c.k = kq_split(R.hdr, L, T == T_Q5_K ? 31.0f : 15.0f);
        (void)u;
    } else if constexpr (T == T_Q6_K) {
        c.k = q6_tile(R, g);
        (void)u;
    } else if constexpr (T == T_FP8) {
        // code * s * 2^(15-u): at most 4 + 8 significant bits, rounded once
        c.a[0] = bf16_lo(R.sc) * pow2f(15 - u);
        c.a[1] = bf16_hi(R.sc) * pow2f(15 - u);
    } else {
        c = 0;
    }
    (void)L;
    (void)g;
    return c;
}

// Q4_K / Q5_K operand of step s (the exact split's o, kq_split) with the quant dword
// byte-paired first ([b0 b2 b1 b3]), so that its slots hold positions 4s..4s+3 of
// sub-block 2g and then 4s..4s+3 of 2g+1 in order: the x of a step is two runs of
// four, staged without permutes.
template <bool Q5>
__device__ __forceinline__ h8 pkq_step(const MRawKq &R, const KqSplit &K, int g, int s) {
    const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
    const uint32_t w = pair_bytes(qw[s], qw[s], kSelAligned), w8 = w >> 8;
    uint32_t lo01 = w & 0x000F000Fu, lo23 = w8 & 0x000F000Fu;
    uint32_t hi01 = w & 0x00F000F0u, hi23 = w8 & 0x00F000F0u;
    if (Q5) {
        const uint32_t hw[8] = {R.h0.x, R.h0.y, R.h0.z, R.h0.w, R.h1.x, R.h1.y, R.h1.z, R.h1.w};
        q5_fifth(pair_bytes(hw[s], hw[s], kSelAligned) >> (2 * g), lo01, lo23, hi01, hi23);
    }
    return mk_h8(pkfma(lo01, K.s0, K.c0), pkfma(lo23, K.s0, K.c0), pkfma(hi01, K.s1, K.c1), pkfma(hi23, K.s1, K.c1));
}

// The weight operand of step s (0..7) for the types with one step per operand.
template <int T>
__device__ __forceinline__ h8 p_step(const typename MRawOf<T>::type &R, const typename PCoefOf<T>::type &C, int g,
                                     int s) {
    if constexpr (T == T_Q4_K || T == T_Q5_K) {
        return pkq_step<T == T_Q5_K>(R, C.k, g, s);
    } else if constexpr (T == T_FP8) {
        const h8 v = f8_step(R, s);
        const u32x4 w = __builtin_bit_cast(u32x4, v);
        const float a = C.a[s >> 2];
        return mk_h8(mix2(w.x, a, 0.0f), mix2(w.y, a, 0.0f), mix2(w.z, a, 0.0f), mix2(w.w, a, 0.0f));
    } else {
        (void)C;
        (void)g;
        return f4_step(R, s);
    }
}

// x staging.  Half-group q = ((g * BM + t) << 1) | h of the block's x for a
// superblock: token t0 + t (clamped to the last), the x behind units 4h .. 4h+3 of
// lane group g, i.e. four 16-byte loads from p_xsrc(q) + 256 * b halves at the
// offsets xhalf_off, written as units (g * BM + t) * 9 + 4h + i, each unit the two
// 8-byte pieces of step 4h + i in order (the operand order of pkq_step, q6p_steps,
// f4_step and f8_step: no permutes).
template <int T, int BM>
__device__ __forceinline__ const _Float16 *p_xsrc(const PrefillArgs &A, int64_t t0, int q) {
    const int h = q & 1, r = q >> 1, t = r % BM, g = r / BM;
    const int64_t tok = t0 + t < A.n ? t0 + t : A.n - 1;
    return reinterpret_cast<const _Float16 *>(A.x) + tok * A.k + xhalf_base<T>(g, h);
}
template <int T>
__device__ __forceinline__ void p_xcommit(int q, const XHalf &X, uint4 *xs) {
    uint4 *u = xs + (q >> 1) * kUnitsPerTok + 4 * (q & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint2 p0 = xhalf_piece<T>(X, i, 0), p1 = xhalf_piece<T>(X, i, 1);
        u[i] = make_uint4(p0.x, p0.y, p1.x, p1.y);
    }
    if constexpr (T == T_Q4_K || T == T_Q5_K) {   // the sub-block sums, as in xhalf_commit
        const float s0 = hsum16(X.v[0], X.v[1]), s1 = hsum16(X.v[2], X.v[3]);
        reinterpret_cast<float2 *>(xs + (q >> 1) * kUnitsPerTok + kXSumUnit)[q & 1] = make_float2(s0, s1);
    }
}

template <int T, int NT, int NG>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs A) {
    constexpr int BM = 16 * NG, BN = 64 * NT;
    constexpr int HPT = 8 * BM / 256;   // x half-groups per thread and superblock
    static_assert(HPT >= 1 && (8 * BM) % 256 == 0, "token block too small");
    typedef typename MRawOf<T>::type Raw;
    typedef typename PCoefOf<T>::type Coef;
    extern __shared__ uint4 lds[];   // the block's x for one superblock: 4 * BM * 9 units

    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);   // row group
    const int j = lane & 15, g = lane >> 4;
    // One-dimensional grid, row blocks fastest.
    const int64_t rblocks = (A.m + BN - 1) / BN;
    const int64_t t0 = (int64_t)blockIdx.x / rblocks * BM;
    const int64_t r0 = (int64_t)blockIdx.x % rblocks * BN + wq * (16 * NT);
    const int nb = A.k / 256;

    constexpr int S = T == T_Q4_K ? 144 : (T == T_Q5_K ? 176 : (T == T_Q6_K ? 210 : 0));
    const int sbs = A.tiled ? 16 * S : S;
    const uint8_t *wr[NT];
    const uint8_t *sr[NT];
    int u[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t r = r0 + 16 * i + j, rc = r < A.m ? r : A.m - 1;
        wr[i] = A.tiled ? A.data + (rc >> 4) * (int64_t)nb * 16 * S : A.data + rc * A.row_bytes;
        sr[i] = T == T_NVFP4 ? A.scales + rc * (A.row_bytes / 8)
                             : (T == T_FP8 ? A.scales + (rc >> 7) * (A.row_bytes / 64) : nullptr);
        u[i] = p_row_exp<T>(A, rc);
    }
    const KqLane L = kq_lane_consts(g);
    const _Float16 *xsrc[HPT];
#pragma unroll
    for (int v = 0; v < HPT; ++v) xsrc[v] = p_xsrc<T, BM>(A, t0, tid + 256 * v);

    f4 acc[NT][NG];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int q = 0; q < NG; ++q) acc[i][q] = (f4){0.f, 0.f, 0.f, 0.f};

    // One superblock: the MFMAs of ring slot R over the staged x.
    const uint4 *xl = lds + (g * BM + j) * kUnitsPerTok;   // the lane's token, step 0
    auto compute = [&](Raw (&R)[NT]) __attribute__((always_inline)) {
        Coef C[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            if constexpr (T == T_Q6_K) {
                if (__builtin_amdgcn_ballot_w64(R[i].mis != 0)) q6_extras(R[i], g);   // wave-uniform
            }
            C[i] = p_coef<T>(R[i], L, g, u[i]);
        }
        if constexpr (T == T_Q6_K) {
            // One chain per superblock: y += d*2^16 * sum(o*x) (q6_tile, q6_steps).
            f4 c1[NT][NG];
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int q = 0; q < NG; ++q) c1[i][q] = (f4){0.f, 0.f, 0.f, 0.f};
            auto dword = [&](auto I) __attribute__((always_inline)) {
                constexpr int II = decltype(I)::value;
                h8 xa0[NG], xa1[NG];
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    xa0[q] = u4h8(xl[16 * q * kUnitsPerTok + 2 * II]);
                    xa1[q] = u4h8(xl[16 * q * kUnitsPerTok + 2 * II + 1]);
                }
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    h8 b0, b1;
                    q6_steps<II>(R[i], C[i].k, b0, b1);
#pragma unroll
                    for (int q = 0; q < NG; ++q) {
                        c1[i][q] = mfma(xa0[q], b0, c1[i][q]);
                        c1[i][q] = mfma(xa1[q], b1, c1[i][q]);
                    }
                }
            };
            dword(std::integral_constant<int, 0>{});
            dword(std::integral_constant<int, 1>{});
            dword(std::integral_constant<int, 2>{});
            dword(std::integral_constant<int, 3>{});
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int q = 0; q < NG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][q][e] = __builtin_fmaf(C[i].k.d, c1[i][q][e], acc[i][q][e]);
        } else if constexpr (T == T_Q4_K || T == T_Q5_K) {
            // One chain per superblock: y += d*2^14 * sum(o*x) + sum_j r_j * X_j.
            f4 c1[NT][NG];
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int q = 0; q < NG; ++q) c1[i][q] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                h8 xa[NG];
#pragma unroll
                for (int q = 0; q < NG; ++q) xa[q] = u4h8(xl[16 * q * kUnitsPerTok + s]);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const h8 b = p_step<T>(R[i], C[i], g, s);
#pragma unroll
                    for (int q = 0; q < NG; ++q) c1[i][q] = mfma(xa[q], b, c1[i][q]);
                }
            }
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const uint4 xp = xl[16 * q * kUnitsPerTok + kXSumUnit];
                const float x0 = __builtin_bit_cast(float, xp.x) + __builtin_bit_cast(float, xp.z);
                const float x1 = __builtin_bit_cast(float, xp.y) + __builtin_bit_cast(float, xp.w);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][q][e] = __builtin_fmaf(C[i].k.dd, c1[i][q][e], acc[i][q][e]);
                    acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(x0, C[i].k.r0, acc[i][q], 0, 0, 0);
                    acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(x1, C[i].k.r1, acc[i][q], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                h8 xa[NG];
#pragma unroll
                for (int q = 0; q < NG; ++q) xa[q] = u4h8(xl[16 * q * kUnitsPerTok + s]);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const h8 b = p_step<T>(R[i], C[i], g, s);
#pragma unroll
                    for (int q = 0; q < NG; ++q) acc[i][q] = mfma(xa[q], b, acc[i][q]);
                }
            }
        }
    };
    auto load_w = [&](Raw (&R)[NT], int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NT; ++i) R[i] = mload<T>(wr[i], sr[i], b, g, sbs, A.tiled);
    };
    // x of superblock b: loads into registers, then (after a barrier) into LDS.
    auto fetch_x = [&](XHalf (&X)[HPT], int b) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < HPT; ++v) {
            const _Float16 *p = xsrc[v] + (int64_t)b * 256;
#pragma unroll
            for (int l = 0; l < 4; ++l) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(p + xhalf_off<T>(l));
                X[v].v[l] = make_uint4(w.x, w.y, w.z, w.w);
            }
        }
    };
    auto commit_x = [&](const XHalf (&X)[HPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < HPT; ++v) p_xcommit<T>(tid + 256 * v, X[v], lds);
    };

    // Per superblock b: b+1's weights and x go out, b is computed, barrier, b+1's x
    // is written to LDS, barrier.
    Raw ring0[NT], ring1[NT];
    XHalf X[HPT];
    load_w(ring0, 0);
    fetch_x(X, 0);
    commit_x(X);
    __syncthreads();
    // Two superblocks per trip so that the ring slots are compile-time.
    for (int b = 0; b < nb; b += 2) {
        if (b + 1 < nb) {
            load_w(ring1, b + 1);
            fetch_x(X, b + 1);
        }
        compute(ring0);
        __syncthreads();
        if (b + 1 >= nb) break;   // uniform
        commit_x(X);
        __syncthreads();
        if (b + 2 < nb) {
            load_w(ring0, b + 2);
            fetch_x(X, b + 2);
        }
        compute(ring1);
        __syncthreads();
        if (b + 2 >= nb) break;
        commit_x(X);
        __syncthreads();
    }

    // D tile (i, q): lane holds tokens 16q + 4g + e, weight row 16i + j of the wave's rows.
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t r = r0 + 16 * i + j;
        const float back = p_scaled<T>() ? pow2f(u[i] - 15) : 1.0f;   // exact
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = t0 + 16 * q + 4 * g + e;
                if (t < A.n && r < A.m) A.y[t * A.m + r] = acc[i][q][e] * back;
            }
    }
}

template <int T, int NT, int NG>
static hipError_t launch_cfg(const PrefillArgs &A, hipStream_t st) {
    constexpr int BM = 16 * NG, BN = 64 * NT;
    const int64_t blocks = (A.m + BN - 1) / BN * ((A.n + BM - 1) / BM);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)4 * BM * kUnitsPerTok * 16;
    const void *fn = (const void *)prefill_kernel<T, NT, NG>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((prefill_kernel<T, NT, NG>), dim3((unsigned)blocks), dim3(256), lds, st, A);
    return hipGetLastError();
}

// 64 tokens x 64 weight rows per workgroup (one row tile per wave, four token
// groups).  Measured at 512 tokens against 128 x 128, 128 x 64 and 64 x 128 blocks of
// the same kernel (Q4_K 9728x2560 / Q6_K 2560x9728 / Q5_K 4096x2560, µs): 64.6 /
// 102.8 / 35.5 against 66.8 / 139.0 / 38.5 (64 x 128) and 82.0 / 134.0 / 40.0
// (128 x 64): the small block keeps up to three workgroups per CU busy (at most 160
// VGPRs, 37 KB of LDS), and the larger ones spill registers or leave CUs idle.
hipError_t launch_prefill(const PrefillArgs &A, hipStream_t st) {
    switch (A.type) {
    case T_Q4_K: return launch_cfg<T_Q4_K, 1, 4>(A, st);
    case T_Q5_K: return launch_cfg<T_Q5_K, 1, 4>(A, st);
    case T_Q6_K: return launch_cfg<T_Q6_K, 1, 4>(A, st);
    case T_FP8: return launch_cfg<T_FP8, 1, 4>(A, st);
    default: return launch_cfg<T_NVFP4, 1, 4>(A, st);
    }
}

}  // namespace qg
