// Device-side decoders for the quantized formats, shared by every kernel of
// libqgemm (the GEMV/rows kernel, the dequant probe and the prefill GEMM), so the
// weights a product consumes are the weights the probe writes.
//
// Formats (reflex-llm kernel notes, K-quant GEMV and uint32-load sections;
// reflex-llm Performance page, Path C and Path E; TandemLLM Kernels page, NVFP4):
//   Q4_K 144 B: fp16 d, fp16 dmin, 12 B of packed 6-bit scale/min, 128 B quants
//               (four 32-byte chunks; chunk c feeds sub-block 2c from its low
//               nibbles and sub-block 2c+1 from its high nibbles).
//   Q5_K 176 B: as Q4_K with 32 B of fifth bits ahead of the quants: bit j of
//               byte l belongs to position l of sub-block j.
//   Q6_K 210 B: 128 B low nibbles, 64 B high 2-bit pairs, 16 int8 scales, fp16 d.
//   NVFP4:      e2m1 codes (low nibble = even element), e4m3 scale per 16.
//
// Unpacking (gfx950): two weights per VALU op.  The dequant probe ORs quants into
// the mantissa of an fp16 constant (the normal-range "magic" form: low nibble
// q -> 1024 + q, high nibble q -> 256 + 4q, recovered exactly by one subtraction;
// Q6_K centres q at 32: (1024 + q) - 1056 or (256 + 4q) - 384 per group).  The
// products (1..32 tokens and prefill) mask the quant in place as an fp16 subnormal
// (q * 2^-24 or q * 2^-20) and scale it with one packed fp16 fma per two weights.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

enum : int { T_Q4_K = 12, T_Q5_K = 13, T_Q6_K = 14, T_NVFP4 = 1001, T_FP8 = 1002 };

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ float f16lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
}

// (a & m) | o in one VALU op.  VOP3 on gfx9 takes no literal operands, so the
// compiler splits the literal-mask form into v_and + v_or; with the mask in an
// SGPR (one scalar operand is allowed) and o in a VGPR, one v_and_or_b32 does it.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(o));
    return d;
}

// Reorder the bytes of a quant dword [b0 b1 b2 b3] to [b0 b2 b1 b3] so that the
// 16-bit lanes of (w & 0x000F000F) hold positions (l, l+1) and those of
// ((w >> 8) & 0x000F000F) hold (l+2, l+3).  With `sel` = kSelMis the same
// instruction also realigns data that starts 2 bytes into `lo` (Q6_K blocks at
// odd 210-byte offsets): logical bytes are then physical bytes 2..5 of {hi:lo}.
constexpr uint32_t kSelAligned = 0x03010200u;
constexpr uint32_t kSelMis = 0x05030402u;
__device__ __forceinline__ uint32_t pair_bytes(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---------------------------------------------------------------------------
// Q4_K / Q5_K header: the two sub-blocks j0 = 2c, j1 = 2c+1 of lane chunk c.
// Per-lane constant selectors, set up once by kq_lane_consts().
struct KqLane {
    uint32_t sel;   // byte gather for the packed 6-bit table
    uint32_t mask;  // 0x3F3F (sub-blocks 0..3) or 0x0F0F (4..7)
    uint32_t shm;   // 0 or 4: where a min's low bits sit in its byte
};

__device__ __forceinline__ KqLane kq_lane_consts(int c) {
    KqLane L;
    if (c < 2) {
        uint32_t j0 = 2 * c, j1 = 2 * c + 1;
        L.sel = j0 | (j1 << 8) | (12u << 16) | (12u << 24);   // 12 selects 0x00
        L.mask = 0x3F3Fu;
        L.shm = 0;
    } else {
        uint32_t j0 = 2 * c - 4, j1 = 2 * c - 3;
        L.sel = (4 + j0) | ((4 + j1) << 8) | (j0 << 16) | (j1 << 24);
        L.mask = 0x0F0Fu;
        L.shm = 4;
    }
    return L;
}

// The packed 6-bit scales and mins of the lane's two sub-blocks 2c, 2c+1: sc has
// sc_2c in bits 0..7 and sc_2c+1 in bits 8..15, mn the same for the mins.
// hdr = the 16 header bytes: .x = d | dmin << 16, .y/.z/.w = scale bytes 0..11.
// For sub-blocks 0..3, scale = low 6 bits of byte j, min = low 6 bits of byte j+4.
// For 4..7: low 4 bits of both come from the nibbles of byte j+4 (scale low,
// min high); their top 2 bits are bits 6..7 of bytes j-4 (scale) and j (min).
__device__ __forceinline__ void kq_scale_min(uint4 hdr, const KqLane &L, uint32_t &sc, uint32_t &mn) {
    const uint32_t t1 = __builtin_amdgcn_perm(hdr.w, hdr.y, L.sel);   // scales
    const uint32_t t2 = __builtin_amdgcn_perm(hdr.w, hdr.z, L.sel);   // mins
    sc = (t1 & L.mask) | ((t1 >> 18) & 0x3030u);
    mn = ((t2 >> L.shm) & L.mask) | ((t2 >> 18) & 0x3030u);
}

// Coefficients of the lane's two sub-blocks (the dequant probe's fp32 weights): a
// weight whose magic value is v = B + s*q (B = 1024, s = 1 for the low sub-block;
// B = 256, s = 4 for the high one) is  a*(v - B) + b  with a = d*sc/s, b = -dmin*m.
struct KqCoef {
    float a0, b0, a1, b1;
};

__device__ __forceinline__ KqCoef kq_coef(uint4 hdr, const KqLane &L) {
    uint32_t sc, mn;
    kq_scale_min(hdr, L, sc, mn);
    float d = f16lo(hdr.x), dmin = f16hi(hdr.x);
    KqCoef k;
    k.a0 = d * (float)(sc & 0xFFu);
    k.a1 = (d * 0.25f) * (float)((sc >> 8) & 0xFFu);
    k.b0 = -dmin * (float)(mn & 0xFFu);
    k.b1 = -dmin * (float)((mn >> 8) & 0xFFu);
    return k;
}

// Exact split of the lane's two sub-blocks of a Q4_K / Q5_K superblock for the matrix
// cores.  With A = d*sc and B = dmin*m (both exact in fp32) and an integer c in
// [0, qmax] (the nearest to B/A, 0 when A = 0), every weight of the sub-block is
//     w = d*sc*q - dmin*m = A*(q - c) + r,    r = A*c - B,
// where A*(q - c) = d * 2^14 * o with o = (q - c)*sc*2^-14 an fp16 value computed
// exactly (|q - c|*sc <= 31*63 < 2^11) by one packed fp16 fma from the quant's
// fp16-subnormal bits: o = v*S + C with v = q*2^-24 (low sub-block) or q*2^-20 (high),
// S = sc*2^10 or sc*2^6, C = -c*sc*2^-14.  As c is the nearest integer to B/A, |r| <=
// |A|/2 and every term is bounded by the weight it belongs to: |r| <= |w| and
// |A*(q - c)| <= 2|w| for q != c (clamping c to [0, qmax] only happens where the two
// terms share a sign), so sums over o*x and r*sum(x) carry rounding errors that
// scale with sum|w||x| whatever cancels inside a weight, and a sub-block of zero
// weights gives o = 0 and r = 0 exactly.
struct KqSplit {
    uint32_t s0, c0, s1, c1;   // packed fp16 S and C of sub-blocks 2c (low nibbles) and 2c+1
    float r0, r1;              // their remainders r
    float dd;                  // d * 2^14
};

__device__ __forceinline__ void kq_split_one(float d, float dmin, uint32_t sc, uint32_t m, float sscale, float qmax,
                                             uint32_t &S, uint32_t &C, float &r) {
    const float a = d * (float)sc, b = dmin * (float)m;   // exact
    float c = __builtin_rintf(b * __builtin_amdgcn_rcpf(a));
    c = __builtin_fminf(__builtin_fmaxf(c, 0.0f), qmax);
    c = a != 0.0f ? c : 0.0f;
    r = __builtin_fmaf(a, c, -b);
    const _Float16 sh = (_Float16)((float)sc * sscale);                        // exact: <= 64512
    const _Float16 ch = (_Float16)(-c * (float)sc * (1.0f / 16384.0f));       // exact: c*sc <= 1953
    S = as_u32((h2){sh, sh});
    C = as_u32((h2){ch, ch});
}

__device__ __forceinline__ KqSplit kq_split(uint4 hdr, const KqLane &L, float qmax) {
    uint32_t sc, mn;
    kq_scale_min(hdr, L, sc, mn);
    const float d = f16lo(hdr.x), dmin = f16hi(hdr.x);
    KqSplit k;
    k.dd = d * 16384.0f;
    kq_split_one(d, dmin, sc & 0xFFu, mn & 0xFFu, 1024.0f, qmax, k.s0, k.c0, k.r0);
    kq_split_one(d, dmin, (sc >> 8) & 0xFFu, (mn >> 8) & 0xFFu, 64.0f, qmax, k.s1, k.c1, k.r1);
    return k;
}

// v*S + C on both fp16 halves, one rounding each (v_pk_fma_f16).
__device__ __forceinline__ uint32_t pkfma(uint32_t v, uint32_t S, uint32_t C) {
    return as_u32(__builtin_elementwise_fma(as_h2(v), as_h2(S), as_h2(C)));
}

// Sum of the sixteen fp16 values in two 16-byte units, in a fixed order (two per
// v_dot2_f32_f16 against ones), in fp32.
__device__ __forceinline__ float hsum16(uint4 a, uint4 b) {
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    float s = 0.0f;
    s = __builtin_amdgcn_fdot2(as_h2(a.x), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(a.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(a.z), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(a.w), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(b.x), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(b.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(b.z), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(b.w), one, s, false);
    return s;
}

// The Q5_K fifth bits of four positions, OR-ed into the subnormal quant pairs of one
// dword: hs = the fifth-bit dword shifted right by 2c (bit 0 of each byte belongs to
// sub-block 2c, bit 1 to 2c+1), in the same byte order as the quant dword the pairs
// came from.  lo_a/hi_a take bytes 0 and 2, lo_b/hi_b bytes 1 and 3.
__device__ __forceinline__ void q5_fifth(uint32_t hs, uint32_t &lo_a, uint32_t &lo_b, uint32_t &hi_a,
                                         uint32_t &hi_b) {
    lo_a = and_or(hs << 4, 0x00100010u, lo_a);
    lo_b = and_or(hs >> 4, 0x00100010u, lo_b);
    hi_a = and_or(hs << 7, 0x01000100u, hi_a);
    hi_b = and_or(hs >> 1, 0x01000100u, hi_b);
}

// Four fp16 pairs of one quant dword of a Q4_K/Q5_K chunk (positions l..l+3):
// lo01/lo23 = 1024 + q (sub-block 2c), hi01/hi23 = 256 + 4q (sub-block 2c+1).
struct Quad {
    uint32_t lo01, lo23, hi01, hi23;
};

__device__ __forceinline__ Quad q4_quad(uint32_t w) {
    uint32_t p = pair_bytes(w, w, kSelAligned);
    uint32_t p8 = p >> 8;
    Quad r;
    r.lo01 = and_or(p, 0x000F000Fu, 0x64006400u);
    r.lo23 = and_or(p8, 0x000F000Fu, 0x64006400u);
    r.hi01 = and_or(p, 0x00F000F0u, 0x5C005C00u);
    r.hi23 = and_or(p8, 0x00F000F0u, 0x5C005C00u);
    return r;
}

// Q5_K: add the fifth bit.  hs = fifth-bit dword already shifted right by 2c and
// byte-paired, so bit 0 of each byte belongs to sub-block 2c, bit 1 to 2c+1.
__device__ __forceinline__ Quad q5_quad(uint32_t w, uint32_t hs) {
    Quad r = q4_quad(w);
    r.lo01 = and_or(hs << 4, 0x00100010u, r.lo01);
    r.lo23 = and_or(hs >> 4, 0x00100010u, r.lo23);
    r.hi01 = and_or(hs << 7, 0x01000100u, r.hi01);
    r.hi23 = and_or(hs >> 1, 0x01000100u, r.hi23);
    return r;
}

// ---------------------------------------------------------------------------
// Q6_K: lane chunk c covers half s = c >> 1 and positions 16h .. 16h+15
// (h = c & 1) of each of the four 32-weight groups g of that half.  For one
// dword (positions l..l+3) of the low-nibble runs A (groups 0, 2) and B (groups
// 1, 3) and of the high-bit run H, build the eight fp16 pairs:
//   groups 0, 1: 1024 + q  (low nibble in bits 0..3, high bits in 4..5);
//   groups 2, 3: 256 + 4q  (low nibble already in bits 4..7, high bits in 8..9),
// so one shift of H serves two groups.  q - 32 is recovered per group by
// subtracting 1056 (resp. 384) times the group's sum of x (see q6_coefs).
struct Q6Oct {
    uint32_t v[4][2];   // [group][pair]
};

__device__ __forceinline__ Q6Oct q6_oct(uint32_t a, uint32_t b, uint32_t hq) {
    // a, b, hq already byte-paired ([b0 b2 b1 b3]).
    const uint32_t a8 = a >> 8, b8 = b >> 8, h8 = hq >> 8;
    const uint32_t h4 = hq << 4, h2 = hq << 2, h84 = h8 << 4, h82 = h8 << 2;
    Q6Oct o;
    o.v[0][0] = and_or(h4, 0x00300030u, and_or(a, 0x000F000Fu, 0x64006400u));
    o.v[0][1] = and_or(h84, 0x00300030u, and_or(a8, 0x000F000Fu, 0x64006400u));
    o.v[1][0] = and_or(h2, 0x00300030u, and_or(b, 0x000F000Fu, 0x64006400u));
    o.v[1][1] = and_or(h82, 0x00300030u, and_or(b8, 0x000F000Fu, 0x64006400u));
    o.v[2][0] = and_or(h4, 0x03000300u, and_or(a, 0x00F000F0u, 0x5C005C00u));
    o.v[2][1] = and_or(h84, 0x03000300u, and_or(a8, 0x00F000F0u, 0x5C005C00u));
    o.v[3][0] = and_or(h2, 0x03000300u, and_or(b, 0x00F000F0u, 0x5C005C00u));
    o.v[3][1] = and_or(h82, 0x03000300u, and_or(b8, 0x00F000F0u, 0x5C005C00u));
    return o;
}

// The same eight pairs without the magic exponent: groups 0, 1 hold q in bits 0..5
// of each 16-bit half (the fp16 subnormal q * 2^-24), groups 2, 3 hold it in bits
// 4..9 (q * 2^-20).
__device__ __forceinline__ Q6Oct q6_sub_oct(uint32_t a, uint32_t b, uint32_t hq) {
    const uint32_t a8 = a >> 8, b8 = b >> 8, h8 = hq >> 8;
    const uint32_t h4 = hq << 4, h2 = hq << 2, h84 = h8 << 4, h82 = h8 << 2;
    Q6Oct o;
    o.v[0][0] = and_or(h4, 0x00300030u, a & 0x000F000Fu);
    o.v[0][1] = and_or(h84, 0x00300030u, a8 & 0x000F000Fu);
    o.v[1][0] = and_or(h2, 0x00300030u, b & 0x000F000Fu);
    o.v[1][1] = and_or(h82, 0x00300030u, b8 & 0x000F000Fu);
    o.v[2][0] = and_or(h4, 0x03000300u, a & 0x00F000F0u);
    o.v[2][1] = and_or(h84, 0x03000300u, a8 & 0x00F000F0u);
    o.v[3][0] = and_or(h2, 0x03000300u, b & 0x00F000F0u);
    o.v[3][1] = and_or(h82, 0x03000300u, b8 & 0x00F000F0u);
    return o;
}

// Packed S, C of a Q6_K group with int8 scale sc for q6_sub_oct values: v*S + C =
// (q - 32)*sc*2^-16 (S = sc*2^8 for groups 0, 1, sc*2^4 for 2, 3; C = -sc*2^-11, exact),
// exact in fp16 while |(q - 32)*sc| <= 2^11 (|sc| <= 64), else rounded once.
__device__ __forceinline__ void q6_sc(float sc, bool hi, uint32_t &S, uint32_t &C) {
    const _Float16 s = (_Float16)(sc * (hi ? 16.0f : 256.0f)), c = (_Float16)(sc * (-1.0f / 2048.0f));
    S = as_u32((h2){s, s});
    C = as_u32((h2){c, c});
}

// Signed 8-bit field at bit `off` of w (an int8 Q6_K scale), as fp32.
__device__ __forceinline__ float i8_at(uint32_t w, int off) {
    return (float)(int32_t)__builtin_amdgcn_sbfe(w, off, 8);
}

// Q6_K group coefficients of lane half h: the int8 scales h, h+2 (in l0) and
// h+4, h+6 (in l1 = the next four bytes).  A weight of group g whose magic value is
// v (q6_oct) is  a_g * (v - B_g),  B_g = 1056 (g < 2) or 384 (g >= 2),
//   a_g = d * sc_g (g < 2) or d * sc_g / 4 (g >= 2).
__device__ __forceinline__ void q6_coefs(uint32_t l0, uint32_t l1, float d, int h, float (&coef)[4]) {
    const int sh = 8 * h;
    coef[0] = d * i8_at(l0, sh);
    coef[1] = d * i8_at(l0, sh + 16);
    coef[2] = (d * 0.25f) * i8_at(l1, sh);
    coef[3] = (d * 0.25f) * i8_at(l1, sh + 16);
}

// ---------------------------------------------------------------------------
// NVFP4: one code byte -> two fp16 values (low nibble first), exact e2m1.
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w, int byte) {
    h2 v;
    switch (byte) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3); break;
    }
    return as_u32(v);
}

// OCP E4M3FN codes: bytes 0, 1 (hi = false) or 2, 3 (hi = true) of w -> fp16 pair,
// lower byte in the low half (exact: every e4m3 value is an fp16 value).
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w, bool hi) {
    return as_u32(hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}

// bf16 bits (the low 16 bits of u) -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// OCP E4M3FN byte `byte` of w -> fp32 (exact).
__device__ __forceinline__ float e4m3_at(uint32_t w, int byte) {
    switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
    }
}

}  // namespace qg
