// Row-invariant weight-streaming product on the matrix cores (gfx950), for
// 1 <= n <= 32 tokens: y[t][r] = sum_k w[r][k] * x[t][k].
//
// Sources: reflex-llm kernel notes (fused K-quant GEMV; batched GEMM: weights
// streamed once for all tokens, y[token*M + row]); TandemLLM Kernels page ("Row
// invariance", "Verify twins", and "NVFP4 matrix products": weights are one operand
// and activations the other operand of the matrix instruction, decoded straight from
// wide loads into operand registers, so 1..16 rows cost one instruction per weight
// tile and 17..32 rows two).
//
// Work split.  K of a tile of 16 weight rows is split into KS phases, phase p
// summing superblocks p, p + KS, ... in increasing order, and the phases' partial
// sums are added in phase order; KS depends only on (type, m, k).  A wave computes
// NP phases, every (KS / NP)-th (NP = 1 at decode sizes; 2 or 4 where more rows per
// workgroup pay), each in accumulators of its own, so the KS / NP waves of a tile,
// which sit in one workgroup, compute the same partials for every NP.
// v_mfma_f32_16x16x32_f16 takes
//   A = x          16 tokens x 32 k   (lane (t, g): token t = lane & 15, k-slots 8g..8g+7)
//   B = W^T        32 k x 16 rows     (lane (j, g): row j = lane & 15, the same k-slots)
//   D[t][j]        lane (j, g) holds tokens 4g .. 4g+3 of row j.
// Lane (j, g) streams chunk g (weights 64g .. 64g+63) of each of its superblocks of
// row j.  The k-slot order inside a step follows the cheapest unpacking of the
// weights; x is staged in LDS in that same order, so no weight needs a permute.
//
// Load order (decode: the whole layer's weights are one cold stream).  Every wave
// issues the loads of the x its superblocks need, then all of its weight loads (up
// to kDepth superblocks; a ring refills behind the computation when a wave has
// more), then writes x to a region of LDS of its own.  Nothing ties a wave's
// start of computation to the other waves: issuing stalls once the memory
// pipeline is full, and a workgroup barrier after the loads, or x staged by some
// waves for all, held whole workgroups until their slowest wave had its data.
//
// Exact operands.  Q4_K/Q5_K: each weight w = A*q - B of a sub-block (A = d*sc,
// B = dmin*m, exact in fp32) is split as w = d*2^14*o + r with c = the integer in
// [0, qmax] nearest B/A (0 where A = 0), the fp16 operand o = (q - c)*sc*2^-14 (exact:
// |q - c|*sc < 2^11) and the per-sub-block remainder r = A*c - B (one fp32 rounding,
// |r| <= |w| for every q of the sub-block).  A superblock's MFMA chain over o is
// scaled by d*2^14 in fp32, and two fp32 MFMAs add r times the sub-block sums of x.
// Nothing subtracts two large rounded sums, so the error of a row scales with
// sum|w||x|, and a sub-block whose weights are all zero (A*q = B) contributes
// exactly zero.  The quant enters one packed fp16 fma per two weights as an fp16
// subnormal (its bits in the low mantissa), so o is formed without any rounding.
// Q6_K: the operand is (q-32)*sc*2^-16, exact for |sc| <= 64 (int8 scales drawn in
// 0..63), otherwise rounded once to fp16 (relative error <= 2^-11); d*2^16 is applied
// in fp32.  NVFP4: e2m1 * e4m3 is exact in fp16 and the MFMA accumulates over all of
// K.  FP8: the code is exact in fp16 and the bf16 block scale is applied in fp32 per
// 128-wide block.
//
// Row invariance.  An output (t, r) is produced by the same instructions for every
// n: its MFMAs see only token t's x (A row t) and row r's weights (B column r);
// tokens >= n are zero A rows that never mix into other rows; the split of K over
// waves and the order of the partials are functions of the weight's shape only.
// The number of token groups (1 for n <= 16, 2 above) only adds instructions for
// the second group.
#pragma once
#include "qg_device.hpp"
#include "qg_kernels.h"
#include "qg_mma_launch.h"

namespace qg {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDepth = kMmaDepth;

// ---------------------------------------------------------------------------
// Raw per-lane loads of one superblock (lane chunk g).  Ordinary (temporal) loads:
// a lane's header and quant loads hit the same 128-byte lines, which must stay in
// the vector L1 between the instructions.
struct MRawKq {
    uint4 hdr, q0, q1, h0, h1;
};
// Q6_K: the three 16-byte runs of the lane's chunk, the dword after each (for
// re-aligning blocks at 2-byte offsets; taken from neighbouring lanes, see
// q6_extras), the scale bytes, d and the offset.
struct MRawQ6 {
    uint4 a, b, h;
    uint32_t a4, b4, h4, s2;
    uint32_t s0, s1, d, mis;
};
struct MRawF4 {
    uint4 q0, q1;
    uint32_t sc;
};
// Block-scaled FP8: the lane's 32 codes of each 128-wide scale block of the
// superblock (bytes 32g .. 32g+31 of block 0 in a0/a1, of block 1 in b0/b1) and the
// two blocks' bf16 scales (block 0 low).
struct MRawF8 {
    uint4 a0, a1, b0, b1;
    uint32_t sc;
};

__device__ __forceinline__ uint4 mld16(const uint8_t *p) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t mld4(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

template <int T>
struct MRawOf {
    typedef MRawKq type;
};
template <>
struct MRawOf<T_Q6_K> {
    typedef MRawQ6 type;
};
template <>
struct MRawOf<T_NVFP4> {
    typedef MRawF4 type;
};
template <>
struct MRawOf<T_FP8> {
    typedef MRawF8 type;
};

// Q6_K blocks sit at 210-byte offsets, so a block may start 2 bytes past a 4-byte
// boundary.  Every load is issued from the 4-byte-aligned address below the data;
// the dword after each run, which the byte-pairing permute needs to realign, is
// the first dword of another lane's run (q6_extras).
// base: the wave's tile, uniform across the wave (rows as stored: its first row's
// superblock 0; tiled layout, tile_chunk in qg_loads.hpp: its chunk 0), off: the
// lane's byte offset from it (rows: (row - first row) * row bytes; tiled: 0), so
// that every load is a uniform base plus a 32-bit lane offset; sbs: bytes from one
// superblock (chunk) to the next.  srow: the lane's scale row (NVFP4, FP8).
template <int T>
__device__ __forceinline__ typename MRawOf<T>::type mload(const uint8_t *base, uint32_t off, const uint8_t *srow,
                                                          int b, int g, int sbs, int tiled) {
    typename MRawOf<T>::type r;
    const uint32_t j = threadIdx.x & 15, L = 16 * (uint32_t)g + j;
    if constexpr (T == T_Q4_K) {
        const uint8_t *blk = base + (int64_t)b * sbs;
        const uint32_t oh = tiled ? 16 * j : off, oq = tiled ? 256 + 16 * L : off + 16 + 32 * (uint32_t)g;
        r.hdr = mld16(blk + oh);
        r.q0 = mld16(blk + oq);
        r.q1 = mld16(blk + oq + (tiled ? 1024 : 16));
    } else if constexpr (T == T_Q5_K) {
        const uint8_t *blk = base + (int64_t)b * sbs;
        const uint32_t oh = tiled ? 16 * j : off, o5 = tiled ? 256 + 16 * j : off + 16;
        const uint32_t oq = tiled ? 768 + 16 * L : off + 48 + 32 * (uint32_t)g;
        r.hdr = mld16(blk + oh);
        r.h0 = mld16(blk + o5);
        r.h1 = mld16(blk + o5 + (tiled ? 256 : 16));
        r.q0 = mld16(blk + oq);
        r.q1 = mld16(blk + oq + (tiled ? 1024 : 16));
    } else if constexpr (T == T_Q6_K) {
        // One set of loads at offsets chosen per layout.  Tiled: aligned runs (the
        // realigning dword is fetched but never used).  Rows: every load issued from the
        // 4-byte-aligned address below the data.  (A per-lane pointer here: the
        // uniform-base form measured slower for this type.)
        const uint8_t *blk = base + off + (int64_t)b * sbs;
        const int s = g >> 1, h = g & 1;
        const int mis = tiled ? 0 : (int)((uintptr_t)blk & 3u);   // 0 or 2
        const int oa = tiled ? 16 * (int)L : 64 * s + 16 * h - mis;
        const int ob = tiled ? 1024 + 16 * (int)L : oa + 32;
        const int oh = tiled ? 2048 + 16 * (int)L : 128 + 32 * s + 16 * h - mis;
        const int os = tiled ? 3072 + 16 * (int)j + 8 * s : 192 + 8 * s - mis;
        const int od = tiled ? 3328 + 2 * (int)j : 208;
        r.mis = (uint32_t)mis;
        r.a = mld16(blk + oa);
        r.b = mld16(blk + ob);
        r.h = mld16(blk + oh);
        const u32x2 s01 = *reinterpret_cast<const u32x2 *>(blk + os);
        r.s0 = s01.x;
        r.s1 = s01.y;
        r.s2 = mld4(blk + os + (mis ? 8 : 4));
        r.d = *reinterpret_cast<const uint16_t *>(blk + od);
    } else if constexpr (T == T_FP8) {
        const uint8_t *c = base + (int64_t)b * 256;
        const uint32_t o = off + 32 * (uint32_t)g;
        r.a0 = mld16(c + o);
        r.a1 = mld16(c + o + 16);
        r.b0 = mld16(c + o + 128);
        r.b1 = mld16(c + o + 144);
        r.sc = mld4(srow + (int64_t)b * 4);   // scale row of the lane's 128-row block
    } else {
        const uint8_t *c = base + (int64_t)b * 128;
        const uint32_t o = off + 32 * (uint32_t)g;
        r.q0 = mld16(c + o);
        r.q1 = mld16(c + o + 16);
        r.sc = mld4(srow + (int64_t)b * 16 + 4 * g);
    }
    (void)L;
    return r;
}

__device__ __forceinline__ h2 h2c(float v) {
    const _Float16 h = (_Float16)v;
    return (h2){h, h};
}
__device__ __forceinline__ uint32_t pk_mul(uint32_t a, h2 b) { return as_u32(as_h2(a) * b); }

__device__ __forceinline__ h8 mk_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(h8, (u32x4){a, b, c, d});
}
__device__ __forceinline__ h8 u4h8(uint4 v) { return mk_h8(v.x, v.y, v.z, v.w); }

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// ---------------------------------------------------------------------------
// x staging.  For token t < n, staged superblock cb and lane group g, eight
// 16-byte units at
//     unit ((cb*4 + g)*n + t)*9 + s
// hold the eight x values of each step s (0..7) in the k-slot order of the weight
// operand; a ninth unit pads the pitch to 144 bytes, which makes the 16 tokens of
// a step read conflict-free.
// Lanes of tokens >= n read a block of zeros at the start of LDS instead (no
// branch, no exec mask).
//
// k-slot order of step s for lane group g (offsets inside the superblock):
//   Q4_K:      64g + 8s + {0, 2, 1, 3, 4, 6, 5, 7}   (steps 0..3: sub-block 2g,
//              4..7: sub-block 2g+1)
//   Q5_K:      64g + {4s, 4s+2, 4s+1, 4s+3, 32+4s, 34+4s, 33+4s, 35+4s}
//   Q6_K:      128(g >> 1) + 16(g & 1) + 4(s >> 1) + 64(s & 1) + {0..3, 32..35}
//   NVFP4:     64g + 8s + 0..7
//   FP8:       128(s >> 2) + 32g + 8(s & 3) + 0..7   (steps 0..3 and 4..7 each stay
//              inside one 128-wide scale block)
// (The prefill GEMM stages x with the same items, in the orders of pkq_step and q6_dword.)
constexpr int kUnitsPerTok = 9;
constexpr int kZeroUnits = 9;
// Q4_K / Q5_K: the ninth unit of (cb, g, t) holds the fp32 sums of x over the lane
// group's two sub-blocks, half by half: {sum over positions 0..15 of sub-block 2g,
// of 2g+1, over positions 16..31 of 2g, of 2g+1} (hsum16 of the two pieces; see
// xp_commit).
constexpr int kXSumUnit = 8;

template <int T>
__device__ __forceinline__ void slot_pieces(int g, int s, int &o0, int &o1) {
    if constexpr (T == T_Q6_K) {
        o0 = 128 * (g >> 1) + 16 * (g & 1) + 4 * (s >> 1) + 64 * (s & 1);
        o1 = o0 + 32;
    } else if constexpr (T == T_NVFP4) {
        o0 = 64 * g + 8 * s;
        o1 = o0 + 4;
    } else if constexpr (T == T_FP8) {
        o0 = 128 * (s >> 2) + 32 * g + 8 * (s & 3);
        o1 = o0 + 4;
    } else {
        o0 = 64 * g + 4 * s;
        o1 = o0 + 32;
    }
}

// Staging by items of 32 bytes.  Lane groups 2gh and 2gh+1 of (staged superblock
// cb, token t) take 256 bytes of x (one run; FP8: two 128-byte lines), eight items
// of two 16-byte pieces each; item i has r2 = i >> 3 = (cb*2 + gh)*n + t and k =
// i & 7, which names its lane group 2gh + xp_ge(k) and its units (see xp_commit).
// Consecutive lanes take consecutive items, so each quad of lanes in a load reads
// one whole 128-byte line.  (Lanes that fetched the four loads of half a unit group
// touched two lines per quad: the 32-token calls staged x 15-20 % slower, the
// lines' lookups and not their bytes setting the pace.)  A lane's items are i0 +
// u*STEP for its passes u; STEP is a multiple of 8, so the lane's k is fixed and its
// r2 advances by the uniform STEP/8, carried over n by XPos.

// Byte offsets of item k inside its record pair's x, and of the record pair gh
// inside the superblock's 512 bytes.
template <int T>
__device__ __forceinline__ uint32_t xp_koff(int k) {
    if constexpr (T == T_FP8) return 256u * (uint32_t)(k >> 2) + 32u * (uint32_t)(k & 3);
    else if constexpr (T == T_Q6_K) return 128u * (uint32_t)(k >> 2) + 16u * (uint32_t)(k & 3);
    else return 32u * (uint32_t)k;
}
// Bytes from an item's first 16-byte piece to its second: adjacent, or for Q6_K the
// 32 positions further on that complete the same two units.
template <int T>
__device__ __forceinline__ constexpr int xp_second() {
    return T == T_Q6_K ? 64 : 16;
}
template <int T>
__device__ __forceinline__ uint32_t xp_gbase(int gh) {
    return (T == T_FP8 ? 128u : 256u) * (uint32_t)gh;
}
template <int T>
__device__ __forceinline__ int xp_ge(int k) {
    if constexpr (T == T_Q6_K) return (k >> 1) & 1;
    else if constexpr (T == T_FP8) return (k >> 1) & 1;
    else return k >> 2;
}
template <int T>
__device__ __forceinline__ int xp_jp(int k) {
    if constexpr (T == T_Q6_K) return 4 * (k & 1) + (k >> 2);   // its first unit (the second: + 2)
    else if constexpr (T == T_FP8) return 2 * (k >> 2) + (k & 1);
    else return k & 3;
}

// r2 = cg*n + t (cg = cb*2 + gh).
struct XPos {
    int t, cg;
};
// r / n by a multiply with the launch's n-th reciprocal (exact for r < 2^16).
__device__ __forceinline__ XPos xpos_of(const MmaArgs &A, int r) {
    const int cg = A.n == 1 ? r : (int)(((uint64_t)(uint32_t)r * A.nmagic) >> 32);
    return {r - cg * A.n, cg};
}
// r2 + d for d = dcg*n + dt, 0 <= dt < n.
__device__ __forceinline__ XPos xpos_step(XPos p, int n, int dt, int dcg) {
    int t = p.t + dt, cg = p.cg + dcg;
    const bool wrap = t >= n;
    t = wrap ? t - n : t;
    cg = wrap ? cg + 1 : cg;
    return {t, cg};
}
// Item (p, k) of staged superblocks cb0 + cb*stride, its two pieces; cg is clamped to
// cgmax (items past the end re-read the last record pair and are not written).
template <int T>
__device__ __forceinline__ void xp_fetch(const MmaArgs &A, XPos p, int cgmax, int cb0, int stride, uint32_t koff,
                                         uint4 &v0, uint4 &v1) {
    const int cg = min(p.cg, cgmax);
    const uint32_t off = (uint32_t)p.t * (uint32_t)(2 * A.k) + (uint32_t)(cb0 + (cg >> 1) * stride) * 512u +
                         xp_gbase<T>(cg & 1) + koff;
    const uint8_t *src = reinterpret_cast<const uint8_t *>(A.x) + off;
    const u32x4 a = *reinterpret_cast<const u32x4 *>(src), b = *reinterpret_cast<const u32x4 *>(src + xp_second<T>());
    v0 = make_uint4(a.x, a.y, a.z, a.w);
    v1 = make_uint4(b.x, b.y, b.z, b.w);
}
// The unit group of item (p, k): record (cb*4 + g)*n + t = (2*cg + (g & 1))*n + t.
template <int T>
__device__ __forceinline__ uint4 *xp_units(uint4 *xu, XPos p, int n, int k) {
    return xu + ((2 * p.cg + xp_ge<T>(k)) * n + p.t) * kUnitsPerTok;
}

// Writes item k's pieces v0, v1 (pieces 2jp, 2jp+1) into its unit group u (if `st`:
// the item exists):
//   Q4_K, NVFP4, FP8: units 2jp, 2jp+1;
//   Q5_K: piece j is the first (j < 4) or second half of units 2(j&3), 2(j&3)+1;
//   Q6_K: the item's two pieces (positions P .. P+7 and P+32 .. P+39 of its lane
//     group, bytes xp_koff and xp_koff + 64 of the record pair) are the first and
//     second runs of units jp and jp + 2 (jp = 4(k&1) + (k>>2));
// each run of four Q4_K / Q5_K positions reordered [x0 x2][x1 x3].  NATURAL (the
// prefill's order of pkq_step): Q4_K and Q5_K both as Q5_K, runs in natural order.
// Q4_K / Q5_K: pieces 2jp, 2jp+1 are positions 16h .. 16h+15 of sub-block 2g + (jp >>
// 1), h = jp & 1, and their hsum16 goes to float 2h + (jp >> 1) of the ninth unit.
template <int T, bool NATURAL = false>
__device__ __forceinline__ void xp_commit(int k, bool st, uint4 v0, uint4 v1, uint4 *u) {
    const int jp = xp_jp<T>(k);
    if constexpr ((T == T_Q4_K || T == T_Q5_K) && NATURAL) {
        const float sum = hsum16(v0, v1);
        if (st) {
            const int s0 = 4 * (jp & 1), half = jp >> 1;
            reinterpret_cast<uint2 *>(u + s0)[half] = make_uint2(v0.x, v0.y);
            reinterpret_cast<uint2 *>(u + s0 + 1)[half] = make_uint2(v0.z, v0.w);
            reinterpret_cast<uint2 *>(u + s0 + 2)[half] = make_uint2(v1.x, v1.y);
            reinterpret_cast<uint2 *>(u + s0 + 3)[half] = make_uint2(v1.z, v1.w);
            reinterpret_cast<float *>(u + kXSumUnit)[2 * (jp & 1) + (jp >> 1)] = sum;
        }
    } else if constexpr (T == T_Q4_K || T == T_Q5_K) {
        // [x0 x1 x2 x3 x4 x5 x6 x7] -> [x0 x2] [x1 x3] [x4 x6] [x5 x7]
        const uint4 w0 = make_uint4(__builtin_amdgcn_perm(v0.y, v0.x, 0x05040100u), __builtin_amdgcn_perm(v0.y, v0.x, 0x07060302u),
                                    __builtin_amdgcn_perm(v0.w, v0.z, 0x05040100u), __builtin_amdgcn_perm(v0.w, v0.z, 0x07060302u));
        const uint4 w1 = make_uint4(__builtin_amdgcn_perm(v1.y, v1.x, 0x05040100u), __builtin_amdgcn_perm(v1.y, v1.x, 0x07060302u),
                                    __builtin_amdgcn_perm(v1.w, v1.z, 0x05040100u), __builtin_amdgcn_perm(v1.w, v1.z, 0x07060302u));
        const float sum = hsum16(v0, v1);
        if (st) {
            if constexpr (T == T_Q4_K) {
                u[2 * jp] = w0;
                u[2 * jp + 1] = w1;
            } else {
                const int s0 = 4 * (jp & 1), half = jp >> 1;
                reinterpret_cast<uint2 *>(u + s0)[half] = make_uint2(w0.x, w0.y);
                reinterpret_cast<uint2 *>(u + s0 + 1)[half] = make_uint2(w0.z, w0.w);
                reinterpret_cast<uint2 *>(u + s0 + 2)[half] = make_uint2(w1.x, w1.y);
                reinterpret_cast<uint2 *>(u + s0 + 3)[half] = make_uint2(w1.z, w1.w);
            }
            reinterpret_cast<float *>(u + kXSumUnit)[2 * (jp & 1) + (jp >> 1)] = sum;
        }
    } else if constexpr (T == T_Q6_K) {
        // v0 = positions P .. P+7, v1 = P+32 .. P+39: the two runs of units jp and jp + 2
        if (st) {
            u[jp] = make_uint4(v0.x, v0.y, v1.x, v1.y);
            u[jp + 2] = make_uint4(v0.z, v0.w, v1.z, v1.w);
        }
    } else {
        if (st) {
            u[2 * jp] = v0;
            u[2 * jp + 1] = v1;
        }
    }
}

// ---------------------------------------------------------------------------
// Q4_K / Q5_K weight operands.  Quant dword l of the lane's chunk holds positions
// 4l..4l+3 of sub-block 2g (low nibbles) and of sub-block 2g+1 (high nibbles).
// Masked in place, each 16-bit half is an fp16 subnormal carrying the quant in its
// mantissa: q * 2^-24 (low nibble, bits 0..3, Q5_K's fifth bit at 4) or q * 2^-20
// (high nibble, bits 4..7, fifth bit at 8); one packed fp16 fma per two weights
// gives the exact operands o = (q - c)*sc*2^-14 of the split w = d*2^14*o + r
// (kq_split).  Q4_K: dwords 2e and 2e+1 give step e (positions 8e..8e+7 of
// sub-block 2g, slots (8e, 8e+2), (8e+1, 8e+3), (8e+4, 8e+6), (8e+5, 8e+7)) from
// their low nibbles and step 4 + e (the same positions of sub-block 2g+1) from their
// high ones; the chain takes steps 0, 4, 1, 5, ... (each dword pair's two steps in
// turn).  Q5_K: step s from dword s alone (q5_step).
typedef KqSplit KqTile;

template <bool Q5>
__device__ __forceinline__ KqTile kq_tile(const MRawKq &R, const KqLane &L) {
    return kq_split(R.hdr, L, Q5 ? 31.0f : 15.0f);
}

// Q4_K step e (HI = false: positions 8e..8e+7 of sub-block 2g) or 4 + e (HI: of 2g+1).
template <bool HI>
__device__ __forceinline__ h8 kq_step(const MRawKq &R, const KqTile &K, int e) {
    const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
    const uint32_t m = HI ? 0x00F000F0u : 0x000F000Fu;
    const uint32_t w0 = qw[2 * e], w1 = qw[2 * e + 1];
    const uint32_t S = HI ? K.s1 : K.s0, C = HI ? K.c1 : K.c0;
    return mk_h8(pkfma(w0 & m, S, C), pkfma((w0 >> 8) & m, S, C), pkfma(w1 & m, S, C), pkfma((w1 >> 8) & m, S, C));
}

// Q5_K step s from quant dword s alone: positions 4s..4s+3 of sub-block 2g, slots
// (4s, 4s+2), (4s+1, 4s+3), then the same of 2g+1 (a Q5_K step built from two
// dwords, as Q4_K's, needs registers the 16-wave kernels do not have).
__device__ __forceinline__ h8 q5_step(const MRawKq &R, const KqTile &K, int g, int s) {
    const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
    const uint32_t w = qw[s], w8 = w >> 8;
    uint32_t lo02 = w & 0x000F000Fu, lo13 = w8 & 0x000F000Fu;
    uint32_t hi02 = w & 0x00F000F0u, hi13 = w8 & 0x00F000F0u;
    // fifth bits: bit 2g (low sub-block) and 2g+1 (high) of qh byte l
    const uint32_t hw[8] = {R.h0.x, R.h0.y, R.h0.z, R.h0.w, R.h1.x, R.h1.y, R.h1.z, R.h1.w};
    q5_fifth(hw[s] >> (2 * g), lo02, lo13, hi02, hi13);
    return mk_h8(pkfma(lo02, K.s0, K.c0), pkfma(lo13, K.s0, K.c0), pkfma(hi02, K.s1, K.c1), pkfma(hi13, K.s1, K.c1));
}

// The prefill's operands: step s from quant dword s alone, byte-paired first ([b0 b2
// b1 b3]), so that its slots hold positions 4s..4s+3 of sub-block 2g and then
// 4s..4s+3 of 2g+1 in order: the x of a step is two runs of four, which the
// prefill's stager writes without permutes (xp_commit, NATURAL).
template <bool Q5>
__device__ __forceinline__ h8 pkq_step(const MRawKq &R, const KqTile &K, int g, int s) {
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

// Q6_K.  Lane chunk g = half h6 = g >> 1, quarter q6 = g & 1 (positions 16*q6 ..
// 16*q6+15 of each of the four 32-weight groups of the half).  Dword i of the
// runs A (groups 0, 2), B (groups 1, 3) and H (high bits) covers positions 4i..4i+3;
// q6_sub_oct gives the quant as an fp16 subnormal, q * 2^-24 for groups 0, 1 and
// q * 2^-20 for groups 2, 3 (byte-paired, positions in natural order).  Step s = 2i + e
// takes groups 2e (pairs 0, 1) and then 2e + 1, positions 4i .. 4i+3 of each.  The
// weight operand is (q - 32)*sc*2^-16 (q6_sc: one packed fma per two weights); the
// superblock's chain is scaled by d*2^16.
struct Q6Tile {
    uint32_t S[4], C[4];
    float d;
};

// The aligned dword after each of the lane's runs A, B, H is the first dword of a
// run another lane of the same row loaded (lane chunk g = 2s + h):
//   after A_g: A_{g+1} (h = 0) or B_{g-1} (h = 1)                   lane ^ 16
//   after B_g: B_{g+1} (g = 0, 2), A_2 (g = 1), H_0 (g = 3)         lane + 16
//   after H_g: H_{g+1} (g = 0..2), scale bytes 0..3 (g = 3, from g = 0)   lane + 16
// Each source lane publishes the one value its requester needs.
__device__ __forceinline__ void q6_extras(MRawQ6 &R, int g) {
    const int lane = (int)(threadIdx.x & 63);
    const int nxt = (lane + 16) & 63;
    R.a4 = (uint32_t)__shfl((int)((g & 1) ? R.a.x : R.b.x), lane ^ 16);
    R.b4 = (uint32_t)__shfl((int)(g == 0 ? R.h.x : (g == 2 ? R.a.x : R.b.x)), nxt);
    R.h4 = (uint32_t)__shfl((int)(g == 0 ? R.s0 : R.h.x), nxt);
}

__device__ __forceinline__ Q6Tile q6_tile(const MRawQ6 &R, int g) {
    const uint32_t l0 = __builtin_amdgcn_alignbyte(R.s1, R.s0, R.mis);
    const uint32_t l1 = __builtin_amdgcn_alignbyte(R.s2, R.s1, R.mis);
    const int sh = 8 * (g & 1);
    // scale of group grp: sub-block 8*h6 + 2*grp + q6 (grp 0, 1 in l0; 2, 3 in l1)
    Q6Tile k;
    q6_sc(i8_at(l0, sh), false, k.S[0], k.C[0]);
    q6_sc(i8_at(l0, sh + 16), false, k.S[1], k.C[1]);
    q6_sc(i8_at(l1, sh), true, k.S[2], k.C[2]);
    q6_sc(i8_at(l1, sh + 16), true, k.S[3], k.C[3]);
    k.d = f16lo(R.d) * 65536.0f;
    return k;
}

// Dword I (and I + 1, for re-alignment) of a 16-byte run followed by its extra dword.
template <int I>
__device__ __forceinline__ uint32_t run_pair(uint4 v, uint32_t extra, uint32_t sel) {
    if constexpr (I == 0) return pair_bytes(v.y, v.x, sel);
    else if constexpr (I == 1) return pair_bytes(v.z, v.y, sel);
    else if constexpr (I == 2) return pair_bytes(v.w, v.z, sel);
    else return pair_bytes(extra, v.w, sel);
}

// The two steps 2I, 2I+1 of dword I.
template <int I>
__device__ __forceinline__ void q6_steps(const MRawQ6 &R, const Q6Tile &K, h8 &b0, h8 &b1) {
    const uint32_t sel = R.mis ? kSelMis : kSelAligned;
    const Q6Oct o = q6_sub_oct(run_pair<I>(R.a, R.a4, sel), run_pair<I>(R.b, R.b4, sel), run_pair<I>(R.h, R.h4, sel));
    b0 = mk_h8(pkfma(o.v[0][0], K.S[0], K.C[0]), pkfma(o.v[0][1], K.S[0], K.C[0]), pkfma(o.v[1][0], K.S[1], K.C[1]),
               pkfma(o.v[1][1], K.S[1], K.C[1]));
    b1 = mk_h8(pkfma(o.v[2][0], K.S[2], K.C[2]), pkfma(o.v[2][1], K.S[2], K.C[2]), pkfma(o.v[3][0], K.S[3], K.C[3]),
               pkfma(o.v[3][1], K.S[3], K.C[3]));
}

// NVFP4 step s: codes 8s .. 8s+7 of the lane's 64 (low nibble first), scale s >> 1.
__device__ __forceinline__ h8 f4_step(const MRawF4 &R, int s) {
    const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
    const h2 S = h2c(e4m3_at(R.sc, s >> 1));   // e4m3 values are exact in fp16
    return mk_h8(pk_mul(fp4_pair(qw[s], 0), S), pk_mul(fp4_pair(qw[s], 1), S), pk_mul(fp4_pair(qw[s], 2), S),
                 pk_mul(fp4_pair(qw[s], 3), S));
}

// FP8 step s: the lane's codes 8(s & 3) .. 8(s & 3) + 7 of scale block s >> 2 (exact
// fp16); the block's bf16 scale is applied in fp32 after its four MFMAs.
__device__ __forceinline__ h8 f8_step(const MRawF8 &R, int s) {
    const uint4 v = (s >> 2) ? ((s & 2) ? R.b1 : R.b0) : ((s & 2) ? R.a1 : R.a0);
    const uint32_t w0 = (s & 1) ? v.z : v.x, w1 = (s & 1) ? v.w : v.y;
    return mk_h8(fp8_pair(w0, false), fp8_pair(w0, true), fp8_pair(w1, false), fp8_pair(w1, true));
}

template <int I, int NG>
__device__ __forceinline__ void q6_dword(const MRawQ6 &R, const Q6Tile &K, const uint4 *const (&xv)[NG], f4 (&c1)[NG]) {
    h8 b0, b1;
    q6_steps<I>(R, K, b0, b1);
#pragma unroll
    for (int q = 0; q < NG; ++q) {
        c1[q] = mfma(u4h8(xv[q][2 * I]), b0, c1[q]);
        c1[q] = mfma(u4h8(xv[q][2 * I + 1]), b1, c1[q]);
    }
}

// ---------------------------------------------------------------------------
// One superblock of NT weight tiles for NG token groups.  xa[q] = the lane's nine
// units of the superblock for token group q (or the zeros), read up front.
template <int T, int NT, int NG, bool PAIRED = false>
__device__ __forceinline__ void msb(const typename MRawOf<T>::type (&R)[NT], int g, const KqLane &L, const uint4 *const (&xa)[NG],
                                    f4 (&acc)[NT][NG]) {
    const uint4 *const(&xv)[NG] = xa;   // LDS reads at their use; other waves hide the latency
    if constexpr (T == T_Q4_K || T == T_Q5_K) {
        // c = sum_k o*x over the superblock (one MFMA chain); y += d*2^14 * c, then
        // y += sum_j r_j * X_j over the eight sub-blocks j (X_j = sum of x over
        // sub-block j, staged beside x) with two fp32 MFMAs: lane group g holds the
        // r and X of sub-blocks 2g (first) and 2g+1 (second).
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const KqTile K = kq_tile<T == T_Q5_K>(R[i], L);
            f4 c1[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) c1[q] = (f4){0.f, 0.f, 0.f, 0.f};
            if constexpr (PAIRED) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const h8 b = pkq_step<T == T_Q5_K>(R[i], K, g, s);
#pragma unroll
                    for (int q = 0; q < NG; ++q) c1[q] = mfma(u4h8(xv[q][s]), b, c1[q]);
                }
            } else if constexpr (T == T_Q5_K) {
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const h8 b = q5_step(R[i], K, g, s);
#pragma unroll
                    for (int q = 0; q < NG; ++q) c1[q] = mfma(u4h8(xv[q][s]), b, c1[q]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const h8 blo = kq_step<false>(R[i], K, e);
#pragma unroll
                    for (int q = 0; q < NG; ++q) c1[q] = mfma(u4h8(xv[q][e]), blo, c1[q]);
                    const h8 bhi = kq_step<true>(R[i], K, e);
#pragma unroll
                    for (int q = 0; q < NG; ++q) c1[q] = mfma(u4h8(xv[q][4 + e]), bhi, c1[q]);
                }
            }
#pragma unroll
            for (int q = 0; q < NG; ++q) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][q][e] = __builtin_fmaf(K.dd, c1[q][e], acc[i][q][e]);
                const uint4 xp = xv[q][kXSumUnit];
                const float x0 = __builtin_bit_cast(float, xp.x) + __builtin_bit_cast(float, xp.z);
                const float x1 = __builtin_bit_cast(float, xp.y) + __builtin_bit_cast(float, xp.w);
                acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(x0, K.r0, acc[i][q], 0, 0, 0);
                acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(x1, K.r1, acc[i][q], 0, 0, 0);
            }
        }
    } else if constexpr (T == T_Q6_K) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            MRawQ6 Ri = R[i];
            if (__builtin_amdgcn_ballot_w64(Ri.mis != 0)) q6_extras(Ri, g);   // wave-uniform
            const Q6Tile K = q6_tile(Ri, g);
            f4 c1[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) c1[q] = (f4){0.f, 0.f, 0.f, 0.f};
            q6_dword<0, NG>(Ri, K, xv, c1);
            q6_dword<1, NG>(Ri, K, xv, c1);
            q6_dword<2, NG>(Ri, K, xv, c1);
            q6_dword<3, NG>(Ri, K, xv, c1);
#pragma unroll
            for (int q = 0; q < NG; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][q][e] = __builtin_fmaf(K.d, c1[q][e], acc[i][q][e]);
        }
    } else if constexpr (T == T_FP8) {
        // c = sum over one 128-wide scale block of code*x; y += scale*c per block.
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f4 c1[NG];
#pragma unroll
                for (int q = 0; q < NG; ++q) c1[q] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 4 * h; s < 4 * h + 4; ++s) {
                    const h8 b = f8_step(R[i], s);
#pragma unroll
                    for (int q = 0; q < NG; ++q) c1[q] = mfma(u4h8(xv[q][s]), b, c1[q]);
                }
                const float sc = h ? bf16_hi(R[i].sc) : bf16_lo(R[i].sc);
#pragma unroll
                for (int q = 0; q < NG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][q][e] = __builtin_fmaf(sc, c1[q][e], acc[i][q][e]);
            }
    } else {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const h8 b = f4_step(R[i], s);
#pragma unroll
                for (int q = 0; q < NG; ++q) acc[i][q] = mfma(u4h8(xv[q][s]), b, acc[i][q]);
            }
    }
}

// ---------------------------------------------------------------------------
// Staging of x chunk [cb0, cb1) into LDS by the whole workgroup (16*n*cl items,
// IP per thread and pass: two, or one where the accumulators leave no registers).
// `issue` runs between the last pass's x loads and their LDS writes, so loads it
// issues (the first weight superblocks) are in flight while that x arrives; the
// in-order load counter lets the writes wait for x alone.
template <int T, int IP, class F>
__device__ __forceinline__ void x_stage_then(const MmaArgs &A, uint4 *xu, int cb0, int cb1, F &&issue) {
    static_assert(IP == 1 || IP == 2, "one or two items per pass");
    const int n = A.n;
    const int items = 16 * n * (cb1 - cb0);   // > 0
    const int bd = (int)blockDim.x;           // a multiple of 64
    const int tid = (int)threadIdx.x, k = tid & 7;
    const int w64 = 64 * __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cgmax = 2 * (cb1 - cb0) - 1;
    const XPos dstep = xpos_of(A, bd >> 3);   // bd / 8 record pairs per pass step (uniform)
    int q0 = 0;
    for (; q0 + IP * bd < items; q0 += IP * bd) {   // full passes (uniform trip count)
        uint4 v[2 * IP];
        const XPos p = xpos_of(A, (q0 + tid) >> 3);
        uint4 *const u0 = xp_units<T>(xu, p, n, k);
        if constexpr (IP == 2) {
            const XPos p1 = xpos_step(p, n, dstep.t, dstep.cg);
            uint4 *const u1 = xp_units<T>(xu, p1, n, k);
            xp_fetch<T>(A, p, cgmax, cb0, 1, xp_koff<T>(k), v[0], v[1]);
            xp_fetch<T>(A, p1, cgmax, cb0, 1, xp_koff<T>(k), v[IP], v[IP + 1]);
            xp_commit<T>(k, true, v[0], v[1], u0);
            xp_commit<T>(k, true, v[IP], v[IP + 1], u1);
        } else {
            xp_fetch<T>(A, p, cgmax, cb0, 1, xp_koff<T>(k), v[0], v[1]);
            xp_commit<T>(k, true, v[0], v[1], u0);
        }
    }
    // The last pass: each item's loads go out where the wave has items there (a scalar test).
    uint4 v[4];
    const XPos p = xpos_of(A, (q0 + tid) >> 3);
    const XPos p1 = xpos_step(p, n, dstep.t, dstep.cg);
    uint4 *const u0 = xp_units<T>(xu, p, n, k), *const u1 = xp_units<T>(xu, p1, n, k);
    const bool h0 = q0 + w64 < items, h1 = IP == 2 && q0 + bd + w64 < items;
    if (h0) xp_fetch<T>(A, p, cgmax, cb0, 1, xp_koff<T>(k), v[0], v[1]);
    if (h1) xp_fetch<T>(A, p1, cgmax, cb0, 1, xp_koff<T>(k), v[2], v[3]);
    __builtin_amdgcn_sched_barrier(0);
    issue();
    __builtin_amdgcn_sched_barrier(0);
    if (h0) xp_commit<T>(k, q0 + tid < items, v[0], v[1], u0);
    if (h1) xp_commit<T>(k, q0 + bd + tid < items, v[2], v[3], u1);
}
template <int T, int IP>
__device__ __forceinline__ void x_stage(const MmaArgs &A, uint4 *xu, int cb0, int cb1) {
    x_stage_then<T, IP>(A, xu, cb0, cb1, [] {});
}

// The body for one weight type.  The wave serves NT row tiles (`wr[i]`/`sr[i]` = its
// lane's row in tile i and that row's scales) and phases kw, kw + KW, ..., kw + (NP-1)KW
// (KW = KS / NP): its superblocks, in increasing order, are
//     b(i) = kw + i*KW,   i = 0 .. cnt-1,
// superblock i being of phase kw + (i % NP)*KW and adding into acc[i % NP] (kw and KW
// are wave-uniform scalars).
//
// Decode path: when every wave's superblocks fit one round of loads and their x
// fits four staging rounds of two x items per lane, each wave stages its own x (see below).  Otherwise a ring of kDepth superblocks
// refills behind the computation, and x is staged in chunks of A.kc superblocks in
// turn; every wave steps through every chunk (two barriers per step), whether or
// not it has superblocks there, so all waves meet the same barriers.
template <int T, int NT, int NG, int NP, int D>
__device__ __forceinline__ void mma_body(const MmaArgs &A, int KW, int kw, int sbs, int tl, bool dec, int g, int t,
                                         const uint8_t *const (&wr)[NT], const uint32_t (&wo)[NT],
                                         const uint8_t *const (&sr)[NT], uint4 *lds,
                                         f4 (&acc)[NP][NT][NG]) {
    typedef typename MRawOf<T>::type Raw;
    // Ring depth D; unroll U, a multiple of D and of NP, so that ring slots and
    // accumulator sets are compile-time indices.
    constexpr int U = D > NP ? D : NP;
    // x items per thread and staging pass (four phases of two token groups: one).
    constexpr int IP = NP * NG >= 8 ? 1 : 2;
    static_assert(U % D == 0 && U % NP == 0, "ring and phase sets must tile the unroll");
    const int n = A.n, nb = A.nb, kc = A.kc;
    const uint4 *zero = lds;   // kZeroUnits units of zeros
    uint4 *xu = lds + kZeroUnits;
    const int lkw = __builtin_ctz((unsigned)KW);            // KW is a power of two
    const int cnt = kw < nb ? ((nb - 1 - kw) >> lkw) + 1 : 0;   // wave-uniform
    const int maxcnt = (nb + KW - 1) >> lkw;                     // workgroup-uniform (the cnt of kw = 0)
    auto sb = [&](int i) { return kw + i * KW; };
    const int lastb = cnt > 0 ? sb(cnt - 1) : nb - 1;
    const int nchunks = (nb + kc - 1) / kc;
    const int tid = (int)threadIdx.x;
    (void)nchunks;
    // Lanes of tokens >= n read zeros (workgroup staging) or, in the decode path,
    // which meets no barrier after the zeros are written, the wave's own units:
    // their rows of the product are never stored.
    const KqLane L = kq_lane_consts(g);   // K-quant scale-table selectors of the lane group
    // The lane's (g, token) unit group of superblock 0, hoisted out of the loop with
    // two token groups (with one, the kernels that must fit 96 registers compute it
    // in place).
    int lane_units[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) lane_units[q] = (g * n + 16 * q + t) * kUnitsPerTok;
    auto xa_of = [&](int cb, const uint4 *(&xa)[NG], const uint4 *other) {
        const int cbo = cb * 4 * n * kUnitsPerTok;   // uniform
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int tok = 16 * q + t;
            const int lu = NG == 1 ? (g * n + t) * kUnitsPerTok : lane_units[q];
            xa[q] = tok < n ? xu + (lu + cbo) : other;
        }
    };

    if (NP == 1 && dec) {   // (NP > 1: never) the host guarantees maxcnt <= D and 16 * n * maxcnt <= 128 * kMmaDecRounds
        // Each wave stages the x of its own superblocks in a region of its own: its x
        // loads go out ahead of its weight loads, the in-order load counter lets it
        // wait for x alone, and no barrier ties it to the other waves (whose loads,
        // queued in the same memory pipeline, would otherwise set the pace).  Slot 0
        // is issued with x; slot u + 1 goes out just before slot u is computed.
        // Every slot is loaded unconditionally (a slot past the wave's last
        // superblock re-reads superblock `lastb`, a cache hit, and is not used), so
        // the loads outstanding at each wait are known at compile time.
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        xu += wave * (maxcnt * 4 * n * kUnitsPerTok);
        const int hq = 16 * n * cnt;   // this wave's x items (wave-uniform), two per lane and round
        const int cgmax = 2 * cnt - 1;
        const XPos dstep = xpos_of(A, 8);   // eight record pairs per round step
        const int k = lane & 7;
        Raw ring[D][NT];
        int q0 = 0;
        for (; q0 + 128 < hq; q0 += 128) {   // full rounds (several tokens)
            uint4 v[4];
            const XPos p = xpos_of(A, (q0 + lane) >> 3);
            const XPos p1 = xpos_step(p, n, dstep.t, dstep.cg);
            uint4 *const u0 = xp_units<T>(xu, p, n, k), *const u1 = xp_units<T>(xu, p1, n, k);
            xp_fetch<T>(A, p, cgmax, kw, KW, xp_koff<T>(k), v[0], v[1]);
            xp_fetch<T>(A, p1, cgmax, kw, KW, xp_koff<T>(k), v[2], v[3]);
            xp_commit<T>(k, true, v[0], v[1], u0);
            xp_commit<T>(k, true, v[2], v[3], u1);
        }
        {   // the last round, its loads ahead of the first weight loads
            uint4 v[4];
            const XPos p = xpos_of(A, (q0 + lane) >> 3);
            const XPos p1 = xpos_step(p, n, dstep.t, dstep.cg);
            uint4 *const u0 = xp_units<T>(xu, p, n, k), *const u1 = xp_units<T>(xu, p1, n, k);
            const bool h0 = q0 < hq, h1 = q0 + 64 < hq;
            if (h0) xp_fetch<T>(A, p, cgmax, kw, KW, xp_koff<T>(k), v[0], v[1]);
            if (h1) xp_fetch<T>(A, p1, cgmax, kw, KW, xp_koff<T>(k), v[2], v[3]);
#pragma unroll
            for (int i = 0; i < NT; ++i) ring[0][i] = mload<T>(wr[i], wo[i], sr[i], min(kw, lastb), g, sbs, tl);
            // LDS order within a wave: no barrier
            if (h0) xp_commit<T>(k, q0 + lane < hq, v[0], v[1], u0);
            if (h1) xp_commit<T>(k, q0 + 64 + lane < hq, v[2], v[3], u1);
        }
#pragma unroll
        for (int u = 0; u < D; ++u) {
            if (u + 1 < D) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < NT; ++i) ring[u + 1][i] = mload<T>(wr[i], wo[i], sr[i], min(sb(u + 1), lastb), g, sbs, tl);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (u < cnt) {   // scalar branch
                const uint4 *xa[NG];   // the lane's units, computed in place (fewer live registers)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const int tok = 16 * q + t;
                    xa[q] = tok < n ? xu + ((u * 4 + g) * n + tok) * kUnitsPerTok : xu;
                }
                msb<T, NT, NG>(ring[u], g, L, xa, acc[0]);
            }
        }
        return;
    }

    Raw ring[D][NT];
    x_stage_then<T, IP>(A, xu, 0, min(nb, kc), [&] {   // the ring's loads go out behind the first x loads
#pragma unroll
        for (int u = 0; u < D; ++u)
#pragma unroll
            for (int i = 0; i < NT; ++i) ring[u][i] = mload<T>(wr[i], wo[i], sr[i], min(sb(u), lastb), g, sbs, tl);
    });
    __syncthreads();
    int chunk = 0;
    for (int i0 = 0; i0 < cnt; i0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = i0 + u;
            if (it < cnt) {   // scalar branch
                const int b = sb(it);
                while (b >= (chunk + 1) * kc) {   // scalar
                    ++chunk;
                    __syncthreads();
                    x_stage<T, IP>(A, xu, chunk * kc, min(nb, (chunk + 1) * kc));
                    __syncthreads();
                }
                const uint4 *xa[NG];
                xa_of(b - chunk * kc, xa, zero);
                msb<T, NT, NG>(ring[u % D], g, L, xa, acc[u % NP]);
            }
            if (it + D < cnt) {   // refill only with a superblock the wave still serves
#pragma unroll
                for (int i = 0; i < NT; ++i) ring[u % D][i] = mload<T>(wr[i], wo[i], sr[i], min(sb(it + D), lastb), g, sbs, tl);
            }
        }
    }
    // Step through the remaining chunks so every wave meets the same barriers.
    while (chunk + 1 < nchunks) {
        ++chunk;
        __syncthreads();
        x_stage<T, IP>(A, xu, chunk * kc, min(nb, (chunk + 1) * kc));
        __syncthreads();
    }
}

// WV waves per workgroup = WV / KW tile groups x KW waves (KW = KS / NP, each wave
// NP phases).  A tile group serves rows 16u .. 16u+15 of the matrix.  SwiGLU (SW):
// tile groups come in pairs, the gate rows 16u .. 16u+15 and the same rows of the up
// matrix (S.data2); the gate group hands its sums to the up group through LDS, which
// stores silu(gate) * up.  Which wave serves a row never changes the row's
// instructions.
// Single-tile, single-group Q4_K / NVFP4 launches ask for five waves per SIMD (at
// most 96 VGPRs), so that the 4864 waves of a gate/up pair at KS = 4 are all resident
// at once; the others take what their ring of loads needs.
template <int TS, int NG, int NT, int NP>
constexpr int mma_min_waves() {
    return ((TS & ~(TS_Q4 | TS_F4)) == 0 && NG == 1 && NT == 1 && NP == 1) ? 5 : 1;
}

template <int TS, int NG, int WV, int NT, bool SW, int NP>
__global__ __launch_bounds__(64 * WV, (mma_min_waves<TS, NG, NT, NP>())) void mma_kernel(MmaArgs A) {
    static_assert(NT == 1, "one weight tile per wave");
    extern __shared__ uint4 lds[];
    const int bid = (int)blockIdx.x;
    const bool in1 = A.nseg > 1 && bid >= A.seg[1].wg_begin;
    const bool in2 = A.nseg > 2 && bid >= A.seg[2].wg_begin;
    const MSeg S = in2 ? A.seg[2] : (in1 ? A.seg[1] : A.seg[0]);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // scalar
    const int KS = S.ks, KW = KS / NP, lkw = __builtin_ctz((unsigned)KW), tpw = WV >> lkw;
    const int kw = wave & (KW - 1), rt = wave >> lkw;
    // Ring depth: three superblocks with one phase per wave; with several, four (two
    // in 16-wave workgroups, which have 128 registers, and one there with four phases
    // of two token groups, whose accumulators alone take 32 of them).
    // 16-wave instances for two token groups that can hold Q5_K or Q6_K keep two
    // (their decode path never has more than one superblock per wave: 16 * n * count
    // <= 512 with n > 16).
    constexpr int D = NP == 1 ? (((TS & (TS_Q5 | TS_Q6)) && NG == 2 && WV == 16) ? 2 : kDepth)
                              : (WV <= 8 ? 4 : (NP == 4 && NG == 2 ? 1 : 2));
    const int j = lane & 15, g = lane >> 4;
    const int up = SW ? (rt & 1) : 0;   // SwiGLU: 0 for a gate tile group, 1 for an up one
    const int64_t unit = SW ? (int64_t)(bid - S.wg_begin) * (tpw >> 1) + (rt >> 1)
                            : (int64_t)(bid - S.wg_begin) * tpw + rt;
    int rows[NT];   // < m + 16 <= 2^31
    rows[0] = (int)(unit * 16 + j);
    const int n = A.n;
    if (threadIdx.x < kZeroUnits) lds[threadIdx.x] = make_uint4(0, 0, 0, 0);

    const uint8_t *wr[NT];   // the wave's tile (uniform)
    uint32_t wo[NT];         // the lane's offset from it
    const uint8_t *sr[NT];
    // K-quant superblock bytes; in the 16-row tiled layout a tile's chunks (16
    // superblocks each) follow one another from (r/16) * nb * 16 * sbytes.
    const int sbytes = S.type == T_Q4_K ? 144 : (S.type == T_Q5_K ? 176 : (S.type == T_Q6_K ? 210 : 0));
    const int sbs = S.tiled ? 16 * sbytes : sbytes;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int64_t r = rows[i] < S.m ? rows[i] : S.m - 1;   // rows past m read row m-1; results dropped
        // the tile's first row, clamped to the last tile (uniform): r - t0 is in 0..15
        const int64_t t0 = min(rows[i] - (int64_t)j, (int64_t)(S.m - 1) & ~(int64_t)15);
        const bool second = up != 0;
        wr[i] = (second ? S.data2 : S.data) + (S.tiled ? (t0 >> 4) * A.nb * 16 * sbytes : t0 * S.row_bytes);
        wo[i] = S.tiled ? 0u : (uint32_t)((r - t0) * S.row_bytes);
        const uint8_t *sc = second ? S.scales2 : S.scales;
        // NVFP4: one e4m3 scale per 16 weights of the row; FP8: the bf16 scale row
        // of the row's 128-row block (K/128 scales of 2 bytes).
        sr[i] = S.type == T_NVFP4 ? sc + r * (S.row_bytes / 8)
                                  : (S.type == T_FP8 ? sc + (r >> 7) * (S.row_bytes / 64) : nullptr);
    }
    f4 ph[NP][NT][NG];   // one set of accumulators per phase of the wave
#pragma unroll
    for (int a = 0; a < NP; ++a)
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int q = 0; q < NG; ++q) ph[a][i][q] = (f4){0.f, 0.f, 0.f, 0.f};
    if ((TS & TS_Q4) && S.type == T_Q4_K)
        mma_body<T_Q4_K, NT, NG, NP, D>(A, KW, kw, sbs, S.tiled, S.dec != 0, g, j, wr, wo, sr, lds, ph);
    else if ((TS & TS_Q5) && S.type == T_Q5_K)
        mma_body<T_Q5_K, NT, NG, NP, D>(A, KW, kw, sbs, S.tiled, S.dec != 0, g, j, wr, wo, sr, lds, ph);
    else if ((TS & TS_Q6) && S.type == T_Q6_K)
        mma_body<T_Q6_K, NT, NG, NP, D>(A, KW, kw, sbs, S.tiled, S.dec != 0, g, j, wr, wo, sr, lds, ph);
    else if ((TS & TS_F4) && S.type == T_NVFP4)
        mma_body<T_NVFP4, NT, NG, NP, D>(A, KW, kw, sbs, S.tiled, S.dec != 0, g, j, wr, wo, sr, lds, ph);
    else if ((TS & TS_F8) && S.type == T_FP8)
        mma_body<T_FP8, NT, NG, NP, D>(A, KW, kw, sbs, S.tiled, S.dec != 0, g, j, wr, wo, sr, lds, ph);

    // The KS phase partials of a row tile, added in phase order:
    //     y = (((p0 + p1) + p2) + ...) + p(KS-1).
    // Phase p is set p / KW of wave p % KW of the tile.  One wave holding them all adds
    // them in registers; otherwise every wave parks its sets in LDS slots (tile group,
    // phase) and the tile's first wave adds the KS slots in order.
    constexpr int per = NT * NG;   // 16-byte partials per lane
    f4 *part = reinterpret_cast<f4 *>(lds);
    // The lane index again, from the exec mask (nothing to keep alive through the body).
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    f4(&acc)[NT][NG] = ph[0];
    if (KW == 1) {
#pragma unroll
        for (int a = 1; a < NP; ++a)
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int q = 0; q < NG; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][q][e] += ph[a][i][q][e];
    } else {
        __syncthreads();   // every wave is done reading x from LDS
#pragma unroll
        for (int a = 0; a < NP; ++a) {
            const int slot = rt * KS + kw + a * KW;
            if (kw != 0 || a != 0) {
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int q = 0; q < NG; ++q) part[(slot * per + i * NG + q) * 64 + ln] = ph[a][i][q];
            }
        }
        __syncthreads();
        if (kw != 0) return;
        for (int p = 1; p < KS; ++p) {
            const int slot = rt * KS + p;
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const f4 v = part[(slot * per + i * NG + q) * 64 + ln];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[i][q][e] += v[e];
                }
        }
    }
    if (SW) {
        // The waves left hold their tile group's sums (one per group).  LDS from A.xch
        // on is used by nothing else, so the gate sums go there at once.
        f4 *xch = reinterpret_cast<f4 *>(lds + A.xch) + (rt >> 1) * NG * 64 + ln;
        if (!up) {
#pragma unroll
            for (int q = 0; q < NG; ++q) xch[q * 64] = acc[0][q];
        }
        __syncthreads();   // every surviving wave (the first of each tile group) gets here once
        if (!up) return;
        if (rows[0] < S.m) {
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const f4 gs = xch[q * 64];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = 16 * q + 4 * g + e;
                    if (tok < n) {
                        const float gv = gs[e];
                        S.y[(int64_t)tok * S.m + rows[0]] = gv / (1.0f + __expf(-gv)) * acc[0][q][e];
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        float *y = S.y;
        const float *resid = S.resid;
        if (rows[i] < S.m) {
#pragma unroll
            for (int q = 0; q < NG; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tok = 16 * q + 4 * g + e;
                    if (tok < n) {
                        const int64_t o = (int64_t)tok * S.m + rows[i];
                        float v = acc[i][q][e];
                        if (resid) v = resid[o] + v;
                        y[o] = v;
                    }
                }
        }
    }
}

}  // namespace qg
