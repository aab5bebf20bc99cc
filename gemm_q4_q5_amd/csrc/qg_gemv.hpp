// Weight-streaming GEMV / multi-row product (gfx950): loads, per-type updates
// and the kernel template; instantiated by qg_gemv_nt1.hip and qg_gemv_ntn.hip.
//
// What is computed: y[t][r] = sum_k w[r][k] * x[t][k] for quantized W, fp16 x,
// fp32 y (reflex-llm kernel notes, K-quant GEMV and batched-GEMM sections;
// TandemLLM Kernels page, NVFP4 matrix products).
//
// Mapping.  A weight row is served by 4*P lanes of one 64-lane wavefront:
// lane (p, c) takes the 64-weight chunk c (0..3) of superblocks p, p+P, p+2P, ...
// of the row (256-weight blocks for NVFP4), so a wavefront covers 16/P rows and
// every lane streams whole 16-byte vectors.  P depends only on (type, m, k),
// never on the number of tokens, so a row's instruction sequence -- and hence
// its bits -- is the same for 1 and for 32 tokens (TandemLLM Kernels page,
// "Row invariance" and "Verify twins": reduction order fixed by weight shape,
// no atomics, partials added in a fixed order).  x is staged in LDS per chunk
// of superblocks together with per-sub-block sums of x; each lane keeps one fp32
// accumulator per token (reflex-llm kernel notes, batched GEMM: weights streamed
// once for all tokens), and the 4*P partials of a row are combined by a fixed
// butterfly of cross-lane shuffles.
#pragma once
#include "qg_device.hpp"
#include "qg_kernels.h"

namespace qg {

// ---------------------------------------------------------------------------
// Raw per-lane loads of one superblock, one struct per type, kept separate from
// the arithmetic so a lane can have several superblocks in flight.
struct RawKq {
    uint4 hdr, q0, q1, h0, h1;
};
struct RawQ6 {
    uint4 a, b, h;
    uint32_t a4, b4, h4;
    uint2 s01;
    uint32_t s2;
    uint32_t d;
    uint32_t mis;
};
struct RawF4 {
    uint4 q0, q1;
    uint32_t sc;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Weight loads.  Ordinary (temporal) loads on purpose: a lane's two 16-byte
// quant loads and its header load hit the same 128-byte lines, which must stay
// in the vector L1 between the instructions; non-temporal loads made every
// second access go back to L2.
__device__ __forceinline__ uint4 ld16(const uint8_t *p) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8(const uint8_t *p) {
    const u32x2 v = *reinterpret_cast<const u32x2 *>(p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

__device__ __forceinline__ RawKq load_kq(bool q5, const uint8_t *blk, int c) {
    RawKq r;
    r.hdr = ld16(blk);
    if (q5) {
        r.h0 = ld16(blk + 16);
        r.h1 = ld16(blk + 32);
        r.q0 = ld16(blk + 48 + 32 * c);
        r.q1 = ld16(blk + 64 + 32 * c);
    } else {
        r.h0 = r.h1 = make_uint4(0, 0, 0, 0);
        r.q0 = ld16(blk + 16 + 32 * c);
        r.q1 = ld16(blk + 32 + 32 * c);
    }
    return r;
}

// Q6_K blocks sit at 210-byte offsets, so a block may start 2 bytes past a
// 4-byte boundary.  Every load is issued from the 4-byte-aligned address below
// the data, with one extra dword that the byte-pairing permute uses to realign;
// the extra dword is always inside the same block.
__device__ __forceinline__ RawQ6 load_q6(const uint8_t *blk, int c) {
    const int s = c >> 1, h = c & 1;
    const uint32_t mis = (uint32_t)((uintptr_t)blk & 3u);   // 0 or 2
    const uint8_t *base = blk - mis;
    RawQ6 r;
    r.mis = mis;
    const uint8_t *pa = base + 64 * s + 16 * h;
    const uint8_t *pb = pa + 32;
    const uint8_t *ph = base + 128 + 32 * s + 16 * h;
    r.a = ld16(pa);
    r.b = ld16(pb);
    r.h = ld16(ph);
    r.a4 = ld4(mis ? pa + 16 : pa + 12);
    r.b4 = ld4(mis ? pb + 16 : pb + 12);
    r.h4 = ld4(mis ? ph + 16 : ph + 12);
    const uint8_t *ps = base + 192 + 8 * s;
    r.s01 = ld8(ps);
    r.s2 = ld4(mis ? ps + 8 : ps + 4);
    r.d = *reinterpret_cast<const uint16_t *>(blk + 208);
    return r;
}

__device__ __forceinline__ RawF4 load_f4(const uint8_t *codes, const uint8_t *scales, int c) {
    RawF4 r;
    r.q0 = ld16(codes + 32 * c);
    r.q1 = ld16(codes + 32 * c + 16);
    r.sc = ld4(scales + 4 * c);
    return r;
}

// ---------------------------------------------------------------------------
// x in LDS: for each token, the staged superblocks as fp16 pairs
// (pair i = (x[2i], x[2i+1])) and the eight per-sub-block sums of x.  Each
// superblock's 128 pairs occupy 144 dwords: 16 bytes of padding are inserted so
// that the 16-byte reads the lanes of one pass issue together fall into distinct
// LDS bank groups.  The padding follows the type's read pattern:
//   Q4_K / Q5_K / NVFP4 lanes read at pair offsets 32c (+144 per superblock):
//     pad after every 32 pairs;
//   Q6_K lanes read at 64s + 8h: pad after every 64 pairs.
constexpr int kSbDw = 144;    // LDS dwords per staged superblock and token
constexpr int kXsPerSb = 16;  // LDS floats of x sums per staged superblock and token

template <int T>
__device__ __forceinline__ int xpad(int i) {   // pair index in the chunk -> dword offset
    return T == T_Q6_K ? i + ((i >> 6) << 2) + ((i >> 7) << 3) : i + ((i >> 5) << 2);
}

// Q4_K / Q5_K superblock update of one lane for NT tokens.
template <int NT>
__device__ __forceinline__ void compute_kq(bool q5, const RawKq &R, int c, const KqLane &L,
                                           const uint32_t *xw0, const float *xs0, int tstride_w,
                                           int tstride_s, int n, float (&acc)[NT]) {
    const KqCoef cf = kq_coef(R.hdr, L);
    const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
    Quad qd[8];
    if (q5) {
        const uint32_t hw[8] = {R.h0.x, R.h0.y, R.h0.z, R.h0.w, R.h1.x, R.h1.y, R.h1.z, R.h1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            qd[i] = q5_quad(qw[i], pair_bytes(hw[i], hw[i], kSelAligned) >> (2 * c));
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qd[i] = q4_quad(qw[i]);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            const uint4 *xl = reinterpret_cast<const uint4 *>(xw0 + t * tstride_w + 36 * c);
            const uint4 *xh = xl + 4;
            float slo = 0.0f, shi = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 a = xl[j], b = xh[j];
                slo = dot2(qd[2 * j].lo01, a.x, slo);
                slo = dot2(qd[2 * j].lo23, a.y, slo);
                slo = dot2(qd[2 * j + 1].lo01, a.z, slo);
                slo = dot2(qd[2 * j + 1].lo23, a.w, slo);
                shi = dot2(qd[2 * j].hi01, b.x, shi);
                shi = dot2(qd[2 * j].hi23, b.y, shi);
                shi = dot2(qd[2 * j + 1].hi01, b.z, shi);
                shi = dot2(qd[2 * j + 1].hi23, b.w, shi);
            }
            const float2 xsum = *reinterpret_cast<const float2 *>(xs0 + t * tstride_s + 2 * c);
            float a = acc[t];
            a = __builtin_fmaf(cf.a0, __builtin_fmaf(-1024.0f, xsum.x, slo), a);
            a = __builtin_fmaf(cf.b0, xsum.x, a);
            a = __builtin_fmaf(cf.a1, __builtin_fmaf(-256.0f, xsum.y, shi), a);
            a = __builtin_fmaf(cf.b1, xsum.y, a);
            acc[t] = a;
        }
    }
}

// Q6_K superblock update of one lane: half s = c >> 1, positions 16h..16h+15
// (h = c & 1) of the four 32-weight groups of that half.  xs0 holds, per
// 16-position half of each sub-block, the dot2 chain of x alone.
template <int NT>
__device__ __forceinline__ void compute_q6(const RawQ6 &R, int c, const uint32_t *xw0, const float *xs0,
                                           int tstride_w, int tstride_s, int n, float (&acc)[NT]) {
    const int s = c >> 1, h = c & 1;
    const uint32_t sel = R.mis ? kSelMis : kSelAligned;
    const uint32_t av[5] = {R.a.x, R.a.y, R.a.z, R.a.w, R.a4};
    const uint32_t bv[5] = {R.b.x, R.b.y, R.b.z, R.b.w, R.b4};
    const uint32_t hv[5] = {R.h.x, R.h.y, R.h.z, R.h.w, R.h4};
    Q6Oct oc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        oc[i] = q6_oct(pair_bytes(av[i + 1], av[i], sel), pair_bytes(bv[i + 1], bv[i], sel),
                       pair_bytes(hv[i + 1], hv[i], sel));
    const uint32_t l0 = __builtin_amdgcn_alignbyte(R.s01.y, R.s01.x, R.mis);
    const uint32_t l1 = __builtin_amdgcn_alignbyte(R.s2, R.s01.y, R.mis);
    float coef[4];
    q6_coefs(l0, l1, f16lo(R.d), h, coef);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            // x pairs of group g start at position 128s + 32g + 16h (padded).
            const uint32_t *xt = xw0 + t * tstride_w + 68 * s + 8 * h;
            const float *xh = xs0 + t * tstride_s + 8 * s + h;   // half h of sub-block 4s + g
            float a = acc[t];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint4 x0 = *reinterpret_cast<const uint4 *>(xt + 16 * g);
                const uint4 x1 = *reinterpret_cast<const uint4 *>(xt + 16 * g + 4);
                float sg = 0.0f;
                sg = dot2(oc[0].v[g][0], x0.x, sg);
                sg = dot2(oc[0].v[g][1], x0.y, sg);
                sg = dot2(oc[1].v[g][0], x0.z, sg);
                sg = dot2(oc[1].v[g][1], x0.w, sg);
                sg = dot2(oc[2].v[g][0], x1.x, sg);
                sg = dot2(oc[2].v[g][1], x1.y, sg);
                sg = dot2(oc[3].v[g][0], x1.z, sg);
                sg = dot2(oc[3].v[g][1], x1.w, sg);
                a = __builtin_fmaf(coef[g], __builtin_fmaf(g < 2 ? -1056.0f : -384.0f, xh[2 * g], sg), a);
            }
            acc[t] = a;
        }
    }
}

// NVFP4 256-weight block update of one lane: codes 64c .. 64c+63, four groups of
// 16 with one e4m3 scale each.
template <int NT>
__device__ __forceinline__ void compute_f4(const RawF4 &R, int c, const uint32_t *xw0,
                                           int tstride_w, int n, float (&acc)[NT]) {
    const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
    uint32_t v[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[i][j] = fp4_pair(qw[i], j);
    float sc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) sc[g] = e4m3_at(R.sc, g);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            const uint4 *xt = reinterpret_cast<const uint4 *>(xw0 + t * tstride_w + 36 * c);
            float a = acc[t];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint4 x0 = xt[2 * g], x1 = xt[2 * g + 1];
                float sg = 0.0f;
                sg = dot2(v[2 * g][0], x0.x, sg);
                sg = dot2(v[2 * g][1], x0.y, sg);
                sg = dot2(v[2 * g][2], x0.z, sg);
                sg = dot2(v[2 * g][3], x0.w, sg);
                sg = dot2(v[2 * g + 1][0], x1.x, sg);
                sg = dot2(v[2 * g + 1][1], x1.y, sg);
                sg = dot2(v[2 * g + 1][2], x1.z, sg);
                sg = dot2(v[2 * g + 1][3], x1.w, sg);
                a = __builtin_fmaf(sc[g], sg, a);
            }
            acc[t] = a;
        }
    }
}

// ---------------------------------------------------------------------------
// Per-type policies: the raw loads of one superblock for one lane, and the
// lane's update from it.
template <int T>
struct Pol;

template <>
struct Pol<T_Q4_K> {
    typedef RawKq Raw;
    static __device__ __forceinline__ Raw load(const Seg &S, int64_t r, int b, int c) {
        return load_kq(false, S.data + r * S.row_bytes + (int64_t)b * 144, c);
    }
    template <int NT>
    static __device__ __forceinline__ void update(const Raw &R, int c, const KqLane &L, const uint32_t *xw0,
                                                  const float *xs0, int tw, int ts, int n, float (&acc)[NT]) {
        compute_kq<NT>(false, R, c, L, xw0, xs0, tw, ts, n, acc);
    }
};

template <>
struct Pol<T_Q5_K> {
    typedef RawKq Raw;
    static __device__ __forceinline__ Raw load(const Seg &S, int64_t r, int b, int c) {
        return load_kq(true, S.data + r * S.row_bytes + (int64_t)b * 176, c);
    }
    template <int NT>
    static __device__ __forceinline__ void update(const Raw &R, int c, const KqLane &L, const uint32_t *xw0,
                                                  const float *xs0, int tw, int ts, int n, float (&acc)[NT]) {
        compute_kq<NT>(true, R, c, L, xw0, xs0, tw, ts, n, acc);
    }
};

template <>
struct Pol<T_Q6_K> {
    typedef RawQ6 Raw;
    static __device__ __forceinline__ Raw load(const Seg &S, int64_t r, int b, int c) {
        return load_q6(S.data + r * S.row_bytes + (int64_t)b * 210, c);
    }
    template <int NT>
    static __device__ __forceinline__ void update(const Raw &R, int c, const KqLane &, const uint32_t *xw0,
                                                  const float *xs0, int tw, int ts, int n, float (&acc)[NT]) {
        compute_q6<NT>(R, c, xw0, xs0, tw, ts, n, acc);
    }
};

template <>
struct Pol<T_NVFP4> {
    typedef RawF4 Raw;
    static __device__ __forceinline__ Raw load(const Seg &S, int64_t r, int b, int c) {
        return load_f4(S.data + r * S.row_bytes + (int64_t)b * 128,
                       S.scales + r * (S.row_bytes / 8) + (int64_t)b * 16, c);
    }
    template <int NT>
    static __device__ __forceinline__ void update(const Raw &R, int c, const KqLane &, const uint32_t *xw0,
                                                  const float *, int tw, int, int n, float (&acc)[NT]) {
        compute_f4<NT>(R, c, xw0, tw, n, acc);
    }
};

// x staging.  When a chunk of x fits in kXr 16-byte loads per thread, the
// global loads of x are issued before the lane's weight loads and written to
// LDS after them: the load counter retires in order, so x issued ahead of the
// weights can be consumed while the weights are still in flight.  Larger chunks
// are staged completely before any weight load is issued.
constexpr int kXr = 8;   // uint4 of x a thread may hold across the weight loads

struct XPre {
    uint4 v[kXr];
};

// Token and element of flat index i of a chunk of `per_t` elements per token.
template <int NT>
__device__ __forceinline__ void tok_split(int i, int per_t, int &t, int &j) {
    if (NT == 1) {
        t = 0;
        j = i;
    } else {
        t = i / per_t;
        j = i - t * per_t;
    }
}

template <int NT>
__device__ __forceinline__ void x_fetch(const GemvArgs &A, int cb0, int cb1, XPre &xp) {
    const int per_t = (cb1 - cb0) * 32, total = A.n * per_t;
    const uint4 *xg = reinterpret_cast<const uint4 *>(A.x);
#pragma unroll
    for (int q = 0; q < kXr; ++q) {
        const int i = threadIdx.x + 256 * q;
        if (i < total) {
            int t, j;
            tok_split<NT>(i, per_t, t, j);
            xp.v[q] = xg[((int64_t)t * A.k + (int64_t)cb0 * 256) / 8 + j];
        }
    }
}

// Sums of x by the same dot2 chain the quant sums use (so an all-zero run of
// quants cancels exactly against its bias): per 32-position sub-block for
// Q4_K/Q5_K/NVFP4 (16 pairs), per 16-position half sub-block for Q6_K (8 pairs).
template <int T>
struct XSum {
    static constexpr int kPairs = T == T_Q6_K ? 8 : 16;      // pairs per sum
    static constexpr int kPerSb = T == T_Q6_K ? 16 : 8;      // sums per superblock
};

template <int T, int NT>
__device__ __forceinline__ void x_sums(const GemvArgs &A, uint32_t *xw, float *xsum, int cl) {
    constexpr int np = XSum<T>::kPairs, ns = XSum<T>::kPerSb;
    const int tw = A.kc * kSbDw, ts = A.kc * kXsPerSb;
    for (int i = threadIdx.x; i < A.n * cl * ns; i += 256) {
        int t, k;
        tok_split<NT>(i, cl * ns, t, k);
        const uint32_t *src = xw + t * tw + xpad<T>(k * np);
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < np; ++q) s = dot2(0x3C003C00u, src[q], s);
        xsum[t * ts + (k / ns) * kXsPerSb + (k % ns)] = s;
    }
}

template <int T, int NT>
__device__ __forceinline__ void x_commit(const GemvArgs &A, const XPre &xp, uint32_t *xw, float *xsum, int cb0,
                                         int cb1) {
    const int cl = cb1 - cb0, tw = A.kc * kSbDw;
    const int per_t = cl * 32, total = A.n * per_t;
    __syncthreads();   // the previous chunk's readers are done
#pragma unroll
    for (int q = 0; q < kXr; ++q) {
        const int i = threadIdx.x + 256 * q;
        if (i < total) {
            int t, j;
            tok_split<NT>(i, per_t, t, j);
            *reinterpret_cast<uint4 *>(xw + t * tw + xpad<T>(4 * j)) = xp.v[q];
        }
    }
    __syncthreads();
    x_sums<T, NT>(A, xw, xsum, cl);
    __syncthreads();
}

// Whole staging at once (chunks larger than kXr loads per thread).
template <int T, int NT>
__device__ __forceinline__ void x_stage(const GemvArgs &A, uint32_t *xw, float *xsum, int cb0, int cb1) {
    const int cl = cb1 - cb0, tw = A.kc * kSbDw;
    const int per_t = cl * 32, total = A.n * per_t;
    const uint4 *xg = reinterpret_cast<const uint4 *>(A.x);
    __syncthreads();
    for (int i = threadIdx.x; i < total; i += 256) {
        int t, j;
        tok_split<NT>(i, per_t, t, j);
        *reinterpret_cast<uint4 *>(xw + t * tw + xpad<T>(4 * j)) = xg[((int64_t)t * A.k + (int64_t)cb0 * 256) / 8 + j];
    }
    __syncthreads();
    x_sums<T, NT>(A, xw, xsum, cl);
    __syncthreads();
}

// One lane's pass over its superblocks b in [cb0, cb1), b = p (mod P), of row r.
// D superblocks are loaded per round.  The first round is issued before x is
// staged so its memory latency overlaps the staging; with PF the next round is
// issued before the current one is consumed.
template <int T, int NT, int D, bool PF>
__device__ __forceinline__ void chunk_rows(const GemvArgs &A, const Seg &S, int64_t r, bool active, int p, int c,
                                           const KqLane &L, uint32_t *xw, float *xsum, int cb0, int cb1,
                                           bool do_stage, float (&acc)[NT]) {
    typedef Pol<T> Po;
    typedef typename Po::Raw Raw;
    const int P = S.P;
    int b = active ? cb0 + ((p - cb0) & (P - 1)) : cb1;
    const bool early = A.n * (cb1 - cb0) * 32 <= kXr * 256;   // uniform
    XPre xp;
    if (do_stage) {
        if (early)
            x_fetch<NT>(A, cb0, cb1, xp);
        else
            x_stage<T, NT>(A, xw, xsum, cb0, cb1);
    }
    Raw cur[D];
#pragma unroll
    for (int u = 0; u < D; ++u)
        if (b + u * P < cb1) cur[u] = Po::load(S, r, b + u * P, c);
    if (do_stage && early) x_commit<T, NT>(A, xp, xw, xsum, cb0, cb1);
    const int tw = A.kc * kSbDw, ts = A.kc * kXsPerSb;
    while (b < cb1) {
        const int bn = b + D * P;
        Raw nxt[PF ? D : 1];
        if (PF) {
#pragma unroll
            for (int u = 0; u < D; ++u)
                if (bn + u * P < cb1) nxt[u] = Po::load(S, r, bn + u * P, c);
        }
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int rb = b + u * P - cb0;
            if (b + u * P < cb1)
                Po::template update<NT>(cur[u], c, L, xw + rb * kSbDw, xsum + rb * kXsPerSb, tw, ts, A.n, acc);
        }
        if (PF) {
#pragma unroll
            for (int u = 0; u < D; ++u) cur[u] = nxt[PF ? u : 0];
        } else {
#pragma unroll
            for (int u = 0; u < D; ++u)
                if (bn + u * P < cb1) cur[u] = Po::load(S, r, bn + u * P, c);
        }
        b = bn;
    }
}

template <int T, int NT>
__device__ __forceinline__ void chunk_type(const GemvArgs &A, const Seg &S, int64_t r, bool active, int p, int c,
                                           const KqLane &L, uint32_t *xw, float *xsum, int cb0, int cb1,
                                           float (&acc)[NT], float (&acc2)[NT]) {
    constexpr int D = NT == 1 ? kDepth1 : 1;
    constexpr bool PF = NT > 1;
    chunk_rows<T, NT, D, PF>(A, S, r, active, p, c, L, xw, xsum, cb0, cb1, true, acc);
    if (A.mode == MODE_SWIGLU)
        chunk_rows<T, NT, D, PF>(A, A.seg[1], r, active, p, c, L, xw, xsum, cb0, cb1, false, acc2);
}

// TS: bit set of the weight types the instantiation handles (TS_Q4 | ...).
// Sum of a value over the 4P lanes that serve one row, in a fixed tree (the
// same in every kernel, so a row's bits never depend on the launch): DPP
// exchanges inside quads (lanes i^1, then i^2), half-rows (lane 7-i) and rows
// (lane 15-i), then cross-row shuffles.  Each step adds a symmetric partner's
// value, so every lane of the group ends with the same bits.
__device__ __forceinline__ float dpp_add(float v, int step) {
    const int x = __builtin_bit_cast(int, v);
    int o;
    switch (step) {
    case 0: o = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: o = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: o = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: o = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break; // row_mirror
    }
    return v + __builtin_bit_cast(float, o);
}

__device__ __forceinline__ float group_sum(float v, int gl) {
    v = dpp_add(v, 0);
    v = dpp_add(v, 1);
    if (gl > 4) v = dpp_add(v, 2);
    if (gl > 8) v = dpp_add(v, 3);
    if (gl > 16) v += __shfl_xor(v, 16);
    if (gl > 32) v += __shfl_xor(v, 32);
    return v;
}

template <int NT, int TS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs A) {
    extern __shared__ uint4 lds[];
    const int kc = A.kc;
    uint32_t *xw = reinterpret_cast<uint32_t *>(lds);                 // [n][kc*144] padded pairs
    float *xsum = reinterpret_cast<float *>(xw + A.n * kc * kSbDw);   // [n][kc*kXsPerSb]

    // The matrix this workgroup serves (selected without indexing the argument
    // array, which would force it into scratch memory).
    const int bid = (int)blockIdx.x;
    const bool in1 = A.nseg > 1 && bid >= A.seg[1].wg_begin;
    const bool in2 = A.nseg > 2 && bid >= A.seg[2].wg_begin;
    const Seg S = in2 ? A.seg[2] : (in1 ? A.seg[1] : A.seg[0]);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lp = S.lp;
    const int c = lane & 3;
    const int p = (lane >> 2) & (S.P - 1);
    const int grp = lane >> (2 + lp);
    const int64_t r = ((int64_t)(bid - S.wg_begin) * 4 + wave) * (16 >> lp) + grp;
    const bool active = r < S.m;
    const KqLane L = kq_lane_consts(c);
    const int n = A.n;

    float acc[NT], acc2[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = acc2[t] = 0.0f;

    for (int cb0 = 0; cb0 < A.nb; cb0 += kc) {
        const int cb1 = min(A.nb, cb0 + kc);
        if ((TS & TS_Q4) && S.type == T_Q4_K)
            chunk_type<T_Q4_K, NT>(A, S, r, active, p, c, L, xw, xsum, cb0, cb1, acc, acc2);
        else if ((TS & TS_Q5) && S.type == T_Q5_K)
            chunk_type<T_Q5_K, NT>(A, S, r, active, p, c, L, xw, xsum, cb0, cb1, acc, acc2);
        else if ((TS & TS_Q6) && S.type == T_Q6_K)
            chunk_type<T_Q6_K, NT>(A, S, r, active, p, c, L, xw, xsum, cb0, cb1, acc, acc2);
        else if ((TS & TS_F4) && S.type == T_NVFP4)
            chunk_type<T_NVFP4, NT>(A, S, r, active, p, c, L, xw, xsum, cb0, cb1, acc, acc2);
    }

    const int gl = 4 << lp;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            acc[t] = group_sum(acc[t], gl);
            if (A.mode == MODE_SWIGLU) acc2[t] = group_sum(acc2[t], gl);
        }
    }
    if (!active) return;
    if ((lane & (gl - 1)) != 0) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            const int64_t o = (int64_t)t * S.m + r;
            float v = acc[t];
            if (A.mode == MODE_SWIGLU) {
                const float g = v;
                v = g / (1.0f + __expf(-g)) * acc2[t];
            } else if (S.resid) {
                v = S.resid[o] + v;
            }
            S.y[o] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Single-token kernel.  Same per-row arithmetic as gemv_kernel<1> (the same
// update per superblock, in the same order per lane, the same butterfly), laid
// out as straight-line code for the load pipeline:
//   1. x's global loads (uniform trip count, clamped indices),
//   2. every weight load of the lane: exactly D slots, slot u = superblock
//      p + u*P; a slot past the row's end re-reads the row's last superblock
//      (an L1 hit) and is not used,
//   3. x to LDS and its sub-block sums (x landed first: the load counter
//      retires in order, so the weights stay in flight),
//   4. the updates, consuming the slots in order as they land.
template <int T, int D, bool SW>
__device__ __forceinline__ void gemv1_body(const GemvArgs &A, const Seg &S, int64_t r, bool active, int p, int c,
                                           const KqLane &L, uint32_t *xw, float *xsum, float &acc, float &acc2) {
    typedef Pol<T> Po;
    typedef typename Po::Raw Raw;
    const int P = S.P, nb = A.nb;
    const int total = nb * 32;   // uint4 of x
    const uint4 *xg = reinterpret_cast<const uint4 *>(A.x);
    const int tid = (int)threadIdx.x;
    // Eight named values, not an array: an array would be kept in scratch memory
    // across the ordering barrier below.
    const int nq = (total + 255) >> 8;   // uniform: 16-byte x loads per thread
#define QG_XL(q) uint4 xv##q; if (q < nq) xv##q = xg[min(tid + 256 * q, total - 1)];
    QG_XL(0) QG_XL(1) QG_XL(2) QG_XL(3) QG_XL(4) QG_XL(5) QG_XL(6) QG_XL(7)
#undef QG_XL
    static_assert(kXr == 8, "x staging holds eight 16-byte values per thread");
    __builtin_amdgcn_sched_barrier(0);   // x's loads stay ahead of the weight loads
    const int64_t rr = active ? r : 0;
    Raw cur[D], cur2[D];
#pragma unroll
    for (int u = 0; u < D; ++u) cur[u] = Po::load(S, rr, min(p + u * P, nb - 1), c);
    if (SW) {
#pragma unroll
        for (int u = 0; u < D; ++u) cur2[u] = Po::load(A.seg[1], rr, min(p + u * P, nb - 1), c);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load issued before x is written out
    // Unconditional stores (a clamped slot rewrites the last element with its own
    // value): a store under a branch would let the compiler sink its load below
    // the weight loads, where waiting for x would mean waiting for the weights.
#define QG_XS(q) if (q < nq) *reinterpret_cast<uint4 *>(xw + xpad<T>(4 * min(tid + 256 * q, total - 1))) = xv##q;
    QG_XS(0) QG_XS(1) QG_XS(2) QG_XS(3) QG_XS(4) QG_XS(5) QG_XS(6) QG_XS(7)
#undef QG_XS
    __syncthreads();
    x_sums<T, 1>(A, xw, xsum, nb);
    __syncthreads();
    float a1[1] = {0.0f}, a2[1] = {0.0f};
#pragma unroll
    for (int u = 0; u < D; ++u) {
        const int b = p + u * P;
        if (active && b < nb) {
            Po::template update<1>(cur[u], c, L, xw + b * kSbDw, xsum + b * kXsPerSb, 0, 0, 1, a1);
            if (SW) Po::template update<1>(cur2[u], c, L, xw + b * kSbDw, xsum + b * kXsPerSb, 0, 0, 1, a2);
        }
    }
    acc = a1[0];
    acc2 = a2[0];
}

template <int TS, bool SW, int D>
__global__ __launch_bounds__(256) void gemv1_kernel(GemvArgs A) {
    extern __shared__ uint4 lds[];
    uint32_t *xw = reinterpret_cast<uint32_t *>(lds);
    float *xsum = reinterpret_cast<float *>(xw + A.nb * kSbDw);
    const int bid = (int)blockIdx.x;
    const bool in1 = A.nseg > 1 && bid >= A.seg[1].wg_begin;
    const bool in2 = A.nseg > 2 && bid >= A.seg[2].wg_begin;
    const Seg S = in2 ? A.seg[2] : (in1 ? A.seg[1] : A.seg[0]);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lp = S.lp;
    const int c = lane & 3;
    const int p = (lane >> 2) & (S.P - 1);
    const int grp = lane >> (2 + lp);
    const int64_t r = ((int64_t)(bid - S.wg_begin) * 4 + wave) * (16 >> lp) + grp;
    const bool active = r < S.m;
    const KqLane L = kq_lane_consts(c);
    float acc = 0.0f, acc2 = 0.0f;
    if ((TS & TS_Q4) && S.type == T_Q4_K)
        gemv1_body<T_Q4_K, D, SW>(A, S, r, active, p, c, L, xw, xsum, acc, acc2);
    else if ((TS & TS_Q5) && S.type == T_Q5_K)
        gemv1_body<T_Q5_K, D, SW>(A, S, r, active, p, c, L, xw, xsum, acc, acc2);
    else if ((TS & TS_Q6) && S.type == T_Q6_K)
        gemv1_body<T_Q6_K, D, SW>(A, S, r, active, p, c, L, xw, xsum, acc, acc2);
    else if ((TS & TS_F4) && S.type == T_NVFP4)
        gemv1_body<T_NVFP4, D, SW>(A, S, r, active, p, c, L, xw, xsum, acc, acc2);
    const int gl = 4 << lp;
    acc = group_sum(acc, gl);
    if (SW) acc2 = group_sum(acc2, gl);
    if (!active || (lane & (gl - 1)) != 0) return;
    float v = acc;
    if (SW) {
        const float gv = v;
        v = gv / (1.0f + __expf(-gv)) * acc2;
    } else if (S.resid) {
        v = S.resid[r] + v;
    }
    S.y[r] = v;
}

template <int TS, int D>
hipError_t launch_one1(const GemvArgs &A, int grid, size_t lds, hipStream_t st) {
    if (A.mode == MODE_SWIGLU)
        hipLaunchKernelGGL((gemv1_kernel<TS, true, D>), dim3(grid), dim3(256), lds, st, A);
    else
        hipLaunchKernelGGL((gemv1_kernel<TS, false, D>), dim3(grid), dim3(256), lds, st, A);
    return hipGetLastError();
}

template <int D>
hipError_t launch_gemv1_d(const GemvArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    switch (ts) {
    case TS_Q4: return launch_one1<TS_Q4, D>(A, grid, lds, st);
    case TS_Q5: return launch_one1<TS_Q5, D>(A, grid, lds, st);
    case TS_Q6: return launch_one1<TS_Q6, D>(A, grid, lds, st);
    case TS_F4: return launch_one1<TS_F4, D>(A, grid, lds, st);
    case TS_Q4 | TS_Q6: return launch_one1<TS_Q4 | TS_Q6, D>(A, grid, lds, st);
    default: return launch_one1<TS_ALL, D>(A, grid, lds, st);
    }
}

// Launch gemv_kernel<NT, TS> with `lds` bytes of dynamic LDS.
template <int NT, int TS>
hipError_t launch_one(const GemvArgs &A, int grid, size_t lds, hipStream_t st) {
    if (lds > 65536)
        (void)hipFuncSetAttribute((const void *)gemv_kernel<NT, TS>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
    hipLaunchKernelGGL((gemv_kernel<NT, TS>), dim3(grid), dim3(256), lds, st, A);
    return hipGetLastError();
}

}  // namespace qg
