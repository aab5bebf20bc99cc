// Prefill-chunk GEMM on the matrix cores (gfx950): Y[n][m] = X[n][k] . W^T for
// n of any size, W quantized (Q4_K / Q5_K / Q6_K / NVFP4 / FP8).
//
// Reference: reflex-llm Performance page, Path E / E5 -- a tensor-core K-quant
// prefill GEMM whose per-(row, sub-block) scales are decoded once and whose
// dequantized weights serve many tokens.  Here a workgroup owns a block of 16*NG
// tokens by 16*WV*NT weight rows.  Each of its WV waves owns NT row tiles (16 rows
// each) and builds their v_mfma_f32_16x16x32_f16 weight operands in its own
// registers, straight from the streamed superblocks (the same loads and unpacking
// as the 1..32-token product), so a weight is decoded once per token block and
// never passes through LDS.  The block's tokens (fp16) are staged in LDS once per
// superblock, in the operand's k-slot order, and every wave reads them from there.
// Per superblock and step a wave reads NG x fragments and issues NT*NG MFMAs.
//
// The arithmetic of a superblock is the 1..32-token product's (msb): the same exact
// operands, one MFMA chain per superblock (per 128-wide scale block for FP8) scaled
// by its d or block scale, the Q4_K / Q5_K remainders through fp32 MFMAs; only the
// Q4_K / Q5_K quant dwords are byte-paired first, so that x is staged without
// permutes.  No weight is rounded except a Q6_K one with |sc| > 64 (once, to fp16).
//
// Per superblock b: b+1's weights (Q6_K: b+2's) and x are loaded into registers while
// b is computed from one of two LDS x buffers; b+1's x is written to the other; one
// barrier.  Where two workgroups share a CU, one's barrier overlaps the other's MFMAs.
// Where 128-row blocks would leave CUs idle, Q6_K workgroups take 80 rows in two K
// halves whose sums are added in order at the end.  Loads
// past the last token or weight row are clamped to the last one (every address
// stays in bounds); those rows are never stored.  No row-invariance contract
// (TandemLLM Kernels page, "Prefill kernels"): the result is deterministic, but not
// the decode kernel's bits.
#include "qg_loads.hpp"
#include "qg_mma.hpp"
#include "qg_prefill.h"

namespace qg {

template <int T, int NT, int NG, int WV, int DEPTH, int KH>
__global__ __launch_bounds__(64 * WV, (WV <= 8 ? 8 / WV : 1)) void prefill_kernel(PrefillArgs A) {
    // KH K parts: the WV waves are KH groups of TW row-group waves; part h computes
    // superblocks [h*nh, h*nh + nh) of the same rows, stages their x in LDS buffers of its
    // own, and the parts' sums are added in part order at the end (through LDS).
    static_assert(WV % KH == 0 && (KH == 1 || KH == 2), "K parts");
    constexpr int TW = WV / KH;
    constexpr int BM = 16 * NG, BN = 16 * TW * NT, NTH = 64 * TW;   // NTH: threads per part
    // x staging by 32-byte items (xp_koff, xp_gbase, xp_commit): for a superblock the
    // block's x is 16*BM items; thread ptid of a part takes items ptid + NTH*v, v < IPT,
    // item i having record pair r2 = i >> 3 (lane groups 2gh, 2gh+1 of token t: gh = r2 / BM,
    // t = r2 % BM, token t0 + t clamped to the last) and k = i & 7 = ptid & 7, so each
    // quad of lanes reads one whole 128-byte line.  The units are the order of pkq_step
    // (Q4_K, Q5_K: natural runs), q6_dword and the block-scaled steps.
    // Where NTH does not divide the 16*BM items, a thread's items past the end are the
    // block's last record pair again (same k): a duplicate load and an identical LDS
    // write, no branch.
    constexpr int IPT = (16 * BM + NTH - 1) / NTH;
    static_assert(16 * BM >= NTH, "token block too small");
    typedef typename MRawOf<T>::type Raw;
    extern __shared__ uint4 lds[];   // per K part two buffers of the block's x for one superblock, 4 * BM * 9 units each
    constexpr int XU = 4 * BM * kUnitsPerTok;

    const int tid = (int)threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kh = wv / TW, wq = wv % TW;   // K part, row group (uniform)
    const int ptid = tid - 64 * TW * kh;    // thread index within the part
    const int j = lane & 15, g = lane >> 4;
    // One-dimensional grid, row blocks fastest.
    const int64_t rblocks = (A.m + BN - 1) / BN;
    const int64_t t0 = (int64_t)blockIdx.x / rblocks * BM;
    const int64_t r0 = (int64_t)blockIdx.x % rblocks * BN + wq * (16 * NT);
    const int nb = A.k / 256;
    const int nh = (nb + KH - 1) / KH, kb0 = kh * nh;   // superblocks per part (uniform); the part's first
    const int cnt = min(nh, nb - kb0);                   // the part's own count (the last part may have fewer)
    auto sbi = [&](int i) __attribute__((always_inline)) { return min(kb0 + i, nb - 1); };

    constexpr int S = T == T_Q4_K ? 144 : (T == T_Q5_K ? 176 : (T == T_Q6_K ? 210 : 0));
    const int sbs = A.tiled ? 16 * S : S;
    const uint8_t *wr[NT];   // the wave's tile (uniform)
    uint32_t wo[NT];         // the lane's offset from it
    const uint8_t *sr[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t r = r0 + 16 * i + j, rc = r < A.m ? r : A.m - 1;
        const int64_t t0 = min(r0 + 16 * i, (A.m - 1) & ~(int64_t)15);   // uniform; rc - t0 in 0..15
        wr[i] = A.tiled ? A.data + (t0 >> 4) * (int64_t)nb * 16 * S : A.data + t0 * A.row_bytes;
        wo[i] = A.tiled ? 0u : (uint32_t)((rc - t0) * A.row_bytes);
        sr[i] = T == T_NVFP4 ? A.scales + rc * (A.row_bytes / 8)
                             : (T == T_FP8 ? A.scales + (rc >> 7) * (A.row_bytes / 64) : nullptr);
    }
    const KqLane L = kq_lane_consts(g);
    const int k8 = ptid & 7;
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(A.x) + t0 * (int64_t)(2 * A.k);   // uniform
    uint32_t xoff[IPT];   // item v's bytes from xbase, superblock 0 (< 2^27: t < BM, 2k <= 2^21)
    uint4 *xdst[IPT];     // its unit group, buffer 0
#pragma unroll
    for (int v = 0; v < IPT; ++v) {
        const int it = min(ptid + NTH * v, 16 * BM - 8 + k8);   // it & 7 == k8 (NTH % 8 == 0)
        const int r2 = it >> 3, gh = r2 / BM, t = r2 % BM;
        const int tc = t0 + t < A.n ? t : (int)(A.n - 1 - t0);
        xoff[v] = (uint32_t)tc * (uint32_t)(2 * A.k) + xp_gbase<T>(gh) + xp_koff<T>(k8);
        xdst[v] = lds + kh * XU + ((2 * gh + xp_ge<T>(k8)) * BM + t) * kUnitsPerTok;
    }

    f4 acc[NT][NG];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int q = 0; q < NG; ++q) acc[i][q] = (f4){0.f, 0.f, 0.f, 0.f};

    // One superblock (the part's i-th): the MFMAs of ring slot R over the x staged in
    // buffer `buf`; a part with fewer superblocks skips its last step (uniform).
    const uint4 *xl = lds + kh * XU + (g * BM + j) * kUnitsPerTok;   // the lane's token, step 0
    auto compute = [&](Raw (&R)[NT], int buf, int i) __attribute__((always_inline)) {
        if (KH > 1 && i >= cnt) return;
        const uint4 *xa[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q) xa[q] = xl + buf * KH * XU + 16 * q * kUnitsPerTok;
        msb<T, NT, NG, true>(R, g, L, xa, acc);
        // The compiler's interleaving of the MFMAs with the operand construction and
        // the x reads (mode 1): 3-4 % faster at 512 tokens than its default order.
        __builtin_amdgcn_iglp_opt(1);
    };
    auto load_w = [&](Raw (&R)[NT], int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NT; ++i) R[i] = mload<T>(wr[i], wo[i], sr[i], b, g, sbs, A.tiled);
    };
    // x of superblock b: loads into registers, then into LDS.
    auto fetch_x = [&](uint4 (&X)[2 * IPT], int b) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < IPT; ++v) {
            const uint8_t *src = xbase + xoff[v] + (int64_t)b * 512;
            const u32x4 p = *reinterpret_cast<const u32x4 *>(src), q = *reinterpret_cast<const u32x4 *>(src + xp_second<T>());
            X[2 * v] = make_uint4(p.x, p.y, p.z, p.w);
            X[2 * v + 1] = make_uint4(q.x, q.y, q.z, q.w);
        }
    };
    auto commit_x = [&](const uint4 (&X)[2 * IPT], int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < IPT; ++v) xp_commit<T, true>(k8, true, X[2 * v], X[2 * v + 1], xdst[v] + buf * KH * XU);
    };

    uint4 X[2 * IPT];
    if constexpr (DEPTH == 2) {
        // Per superblock b: b+1's weights and x go out, b is computed from x buffer b % 2,
        // b+1's x is written to the other buffer, one barrier.  That buffer was last read
        // by the computation of b-1, which every wave finished before the previous barrier.
        Raw ring0[NT], ring1[NT];
        load_w(ring0, sbi(0));
        fetch_x(X, sbi(0));
        commit_x(X, 0);
        __syncthreads();
        // Two superblocks per trip so that the ring slots and buffers are compile-time.  The
        // loads are unconditional (the superblock index clamped to the last one; a redundant
        // load at the end): loads under a branch make the compiler wait for them at the join.
        // The scheduling barriers keep them ahead of the computation (left alone, the
        // compiler sinks them to its end, which exposes their whole latency).
        for (int b = 0; b < nh; b += 2) {
            __builtin_amdgcn_sched_barrier(0);
            load_w(ring1, sbi(b + 1));
            fetch_x(X, sbi(b + 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(ring0, 0, b);
            if (b + 1 >= nh) break;   // uniform
            commit_x(X, 1);
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            load_w(ring0, sbi(b + 2));
            fetch_x(X, sbi(b + 2));
            __builtin_amdgcn_sched_barrier(0);
            compute(ring1, 1, b + 1);
            if (b + 2 >= nh) break;
            commit_x(X, 0);
            __syncthreads();
        }
    } else {
        // Weights DEPTH superblocks deep: b+DEPTH-1's weights go out while b is computed
        // (x still one ahead, from the L2), so a superblock's HBM latency is covered by
        // DEPTH-1 computations.  b+1's x is fetched before the weights: loads complete in
        // order, and its commit must not wait for the weights just issued.  DEPTH
        // superblocks per trip (ring slots compile-time), the x buffer b % 2 at run time.
        Raw ring[DEPTH][NT];
#pragma unroll
        for (int s = 0; s + 1 < DEPTH; ++s) load_w(ring[s], sbi(s));
        fetch_x(X, sbi(0));
        commit_x(X, 0);
        __syncthreads();
        for (int b = 0; b < nh; b += DEPTH) {
            bool last = false;
#pragma unroll
            for (int s = 0; s < DEPTH; ++s) {
                __builtin_amdgcn_sched_barrier(0);
                fetch_x(X, sbi(b + s + 1));
                load_w(ring[(s + DEPTH - 1) % DEPTH], sbi(b + s + DEPTH - 1));
                __builtin_amdgcn_sched_barrier(0);
                compute(ring[s], (b + s) & 1, b + s);
                if (b + s + 1 >= nh) {   // uniform
                    last = true;
                    break;
                }
                commit_x(X, (b + s + 1) & 1);
                __syncthreads();
            }
            if (last) break;
        }
    }

    if constexpr (KH == 2) {
        // Part 1's sums through LDS (every wave is past its last x read), added to part
        // 0's in that order; part 0 stores.
        __syncthreads();
        float *red = reinterpret_cast<float *>(lds) + wq * (NT * NG * 4 * 64) + lane;
        if (kh == 1) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int q = 0; q < NG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) red[((i * NG + q) * 4 + e) * 64] = acc[i][q][e];
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int q = 0; q < NG; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][q][e] += red[((i * NG + q) * 4 + e) * 64];
    }

    // D tile (i, q): lane holds tokens 16q + 4g + e, weight row 16i + j of the wave's rows.
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t r = r0 + 16 * i + j;
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t t = t0 + 16 * q + 4 * g + e;
                if (t < A.n && r < A.m) A.y[t * A.m + r] = acc[i][q][e];
            }
    }
}

template <int T, int NT, int NG, int WV, int DEPTH, int KH = 1>
static hipError_t launch_cfg(const PrefillArgs &A, hipStream_t st) {
    constexpr int BM = 16 * NG, BN = 16 * (WV / KH) * NT;
    const int64_t blocks = (A.m + BN - 1) / BN * ((A.n + BM - 1) / BM);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const size_t lds = (size_t)2 * KH * 4 * BM * kUnitsPerTok * 16;   // two x buffers per K part
    static_assert((size_t)2 * KH * 4 * BM * kUnitsPerTok * 16 >= (size_t)(WV / KH) * NT * NG * 4 * 64 * 4, "reduction");
    const void *fn = (const void *)prefill_kernel<T, NT, NG, WV, DEPTH, KH>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((prefill_kernel<T, NT, NG, WV, DEPTH, KH>), dim3((unsigned)blocks), dim3(64 * WV), lds, st, A);
    return hipGetLastError();
}

// 64 tokens per workgroup, one 16-row tile per wave and four token groups: 128 weight
// rows in eight waves.  Measured at 512 tokens (Q4_K 9728x2560 / Q6_K 2560x9728 /
// Q5_K 4096x2560, µs): eight waves 61.0 / 88.0 / 31.1 against 62.2 / 89.4 / 33.8 with
// four (each wave's work is the same; a block's x is staged by twice the threads, so
// each holds half as much of it in registers); 128 tokens in eight waves 87.4 / 145.7
// / 46.8; 32 tokens in four 64.5 / 97.8 / 38.9; earlier, two tiles per wave (64 x 128
// in four waves) or 128 tokens in four waves spilled registers or left CUs idle.
// FP8 / NVFP4 (4096 and 16384 rows x 4096, 512 tokens, µs): eight waves 35.2 / 30.4
// and 118 / 95 against 42.4 / 33.3 and 175 / 116 with four.  Weights three superblocks
// deep for Q6_K only (its kernel holds one workgroup per CU either way: 143 -> 177
// VGPRs): 2560x9728 92.0 -> 84.8 µs, 1024x2560 26.8 -> 25.4; four deep 85.5.  For the
// others a third ring slot gains nothing or costs the second workgroup per CU (Q4_K
// 120 -> 149 VGPRs, 63.4 -> 75.2 µs; FP8 16384x4096 114.5 -> 127.3).
constexpr int64_t kPrefillCUs = 256;   // MI355X compute units
hipError_t launch_prefill(const PrefillArgs &A, hipStream_t st) {
    switch (A.type) {
    case T_Q4_K: return launch_cfg<T_Q4_K, 1, 4, 8, 2>(A, st);
    case T_Q5_K: return launch_cfg<T_Q5_K, 1, 4, 8, 2>(A, st);
    case T_Q6_K: {
        // Too few 128-row blocks to fill the chip (the 2560-row down projection: 160
        // workgroups): 80-row blocks in ten waves, five row tiles times two K halves.
        const int64_t tb = (A.n + 63) / 64;
        if (A.k >= 512 && (A.m + 127) / 128 * tb < kPrefillCUs && (A.m + 79) / 80 * tb <= kPrefillCUs)
            return launch_cfg<T_Q6_K, 1, 4, 10, 2, 2>(A, st);
        return launch_cfg<T_Q6_K, 1, 4, 8, 3>(A, st);
    }
    case T_FP8: return launch_cfg<T_FP8, 1, 4, 8, 2>(A, st);
    default: return launch_cfg<T_NVFP4, 1, 4, 8, 2>(A, st);
    }
}

}  // namespace qg
