// Per-lane raw loads of one 64-weight chunk of a quantized superblock, shared by the
// dequant probe (qg_dequant.hip) and the dequantizing stage of the prefill GEMM
// (qg_prefill.hip).  Chunk c of a K-quant superblock is quant bytes 32c .. 32c+31
// (sub-blocks 2c and 2c+1); for Q6_K it is half c >> 1, positions 16(c & 1) ..
// 16(c & 1)+15 of each of its four 32-weight groups; for NVFP4 and FP8, codes
// 64c .. 64c+63 (FP8: with the bf16 scale of the 128-wide block they sit in).
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

struct RawF8 {
    uint4 q0, q1, q2, q3;
    uint32_t sc;   // bf16 scale in the low 16 bits
};

// codes: the superblock's 256 codes; srow: the row's bf16 scale row; b: superblock.
__device__ __forceinline__ RawF8 load_f8(const uint8_t *codes, const uint8_t *srow, int b, int c) {
    RawF8 r;
    r.q0 = ld16(codes + 64 * c);
    r.q1 = ld16(codes + 64 * c + 16);
    r.q2 = ld16(codes + 64 * c + 32);
    r.q3 = ld16(codes + 64 * c + 48);
    r.sc = *reinterpret_cast<const uint16_t *>(srow + (2 * b + (c >> 1)) * 2);
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
// Superblock b of row r of a K-quant matrix of S-byte superblocks, rows one after
// another (the layout as stored).
__device__ __forceinline__ const uint8_t *kq_block(const uint8_t *data, int64_t row_bytes, int S, int64_t r, int b) {
    return data + r * row_bytes + (int64_t)b * S;
}

// The 16-row tiled layout (qg_pack_tiles): superblock b of the 16 rows of tile r/16 is
// one chunk of 16*S bytes at ((r/16 * nb + b) * 16) * S, and inside it every 16-byte
// piece a lane of the product loads is contiguous with its neighbours' (lane L = 16g +
// j: row j of the tile, lane group g), so each load instruction of a wave reads one run
// of bytes:
//   Q4_K (S = 144): header of row j at 16j; quant bytes 32g..32g+15 of row j at
//                   256 + 16L, 32g+16..32g+31 at 1280 + 16L.
//   Q5_K (S = 176): header at 16j; fifth-bit bytes 0..15 at 256 + 16j, 16..31 at
//                   512 + 16j; quant bytes 32g.. at 768 + 16L, 32g+16.. at 1792 + 16L.
//   Q6_K (S = 210): g = 2s + h: low-nibble bytes 64s+16h.. at 16L, 64s+32+16h.. at
//                   1024 + 16L, high-bit bytes 32s+16h.. at 2048 + 16L; the 16 int8
//                   scales of row j at 3072 + 16j; d at 3328 + 2j.
// Every byte of the 16 superblocks appears exactly once; rows past m in a last partial
// tile repeat row m-1.
__device__ __forceinline__ const uint8_t *tile_chunk(const uint8_t *data, int nb, int S, int64_t r, int b) {
    return data + (((r >> 4) * nb + b) * 16) * (int64_t)S;
}

// Byte offset, inside row j's superblock, of byte e (even) of a tiled chunk, and j.
__device__ __forceinline__ int tile_src(int S, int e, int &j) {
    if (S == 144) {
        if (e < 256) { j = e >> 4; return e & 15; }
        const int hi = e >= 1280, L = ((e - (hi ? 1280 : 256)) >> 4);
        j = L & 15;
        return 16 + 32 * (L >> 4) + 16 * hi + (e & 15);
    }
    if (S == 176) {
        if (e < 256) { j = e >> 4; return e & 15; }
        if (e < 768) { const int hi = e >= 512; j = (e - (hi ? 512 : 256)) >> 4; return 16 + 16 * hi + (e & 15); }
        const int hi = e >= 1792, L = ((e - (hi ? 1792 : 768)) >> 4);
        j = L & 15;
        return 48 + 32 * (L >> 4) + 16 * hi + (e & 15);
    }
    // 210
    if (e < 3072) {
        const int run = e >> 10, L = (e & 1023) >> 4, g = L >> 4, s = g >> 1, h = g & 1;
        j = L & 15;
        return (run == 0 ? 64 * s + 16 * h : (run == 1 ? 64 * s + 32 + 16 * h : 128 + 32 * s + 16 * h)) + (e & 15);
    }
    if (e < 3328) { j = (e - 3072) >> 4; return 192 + (e & 15); }
    j = (e - 3328) >> 1;
    return 208 + (e & 1);
}

// Raw loads of chunk c of a tiled superblock (lane group c of row j = r & 15).
__device__ __forceinline__ RawKq load_kq_tiled(bool q5, const uint8_t *ch, int j, int c) {
    const int L = 16 * c + j;
    RawKq r;
    r.hdr = ld16(ch + 16 * j);
    if (q5) {
        r.h0 = ld16(ch + 256 + 16 * j);
        r.h1 = ld16(ch + 512 + 16 * j);
        r.q0 = ld16(ch + 768 + 16 * L);
        r.q1 = ld16(ch + 1792 + 16 * L);
    } else {
        r.h0 = r.h1 = make_uint4(0, 0, 0, 0);
        r.q0 = ld16(ch + 256 + 16 * L);
        r.q1 = ld16(ch + 1280 + 16 * L);
    }
    return r;
}

__device__ __forceinline__ RawQ6 load_q6_tiled(const uint8_t *ch, int j, int c) {
    const int L = 16 * c + j, s = c >> 1;
    RawQ6 r;
    r.mis = 0;
    r.a = ld16(ch + 16 * L);
    r.b = ld16(ch + 1024 + 16 * L);
    r.h = ld16(ch + 2048 + 16 * L);
    r.a4 = r.b4 = r.h4 = 0;   // aligned runs: the realigning dword is never used
    r.s01 = ld8(ch + 3072 + 16 * j + 8 * s);
    r.s2 = 0;
    r.d = *reinterpret_cast<const uint16_t *>(ch + 3328 + 2 * j);
    return r;
}

// The raw chunk type and loader of a weight type (tiled: K-quants only).
template <int T>
struct Loader;

template <>
struct Loader<T_Q4_K> {
    typedef RawKq Raw;
    static __device__ __forceinline__ Raw load(const uint8_t *data, const uint8_t *, int64_t row_bytes, int64_t r,
                                               int b, int c, int tiled) {
        if (tiled) return load_kq_tiled(false, tile_chunk(data, (int)(row_bytes / 144), 144, r, b), (int)(r & 15), c);
        return load_kq(false, kq_block(data, row_bytes, 144, r, b), c);
    }
};

template <>
struct Loader<T_Q5_K> {
    typedef RawKq Raw;
    static __device__ __forceinline__ Raw load(const uint8_t *data, const uint8_t *, int64_t row_bytes, int64_t r,
                                               int b, int c, int tiled) {
        if (tiled) return load_kq_tiled(true, tile_chunk(data, (int)(row_bytes / 176), 176, r, b), (int)(r & 15), c);
        return load_kq(true, kq_block(data, row_bytes, 176, r, b), c);
    }
};

template <>
struct Loader<T_Q6_K> {
    typedef RawQ6 Raw;
    static __device__ __forceinline__ Raw load(const uint8_t *data, const uint8_t *, int64_t row_bytes, int64_t r,
                                               int b, int c, int tiled) {
        if (tiled) return load_q6_tiled(tile_chunk(data, (int)(row_bytes / 210), 210, r, b), (int)(r & 15), c);
        return load_q6(kq_block(data, row_bytes, 210, r, b), c);
    }
};

template <>
struct Loader<T_NVFP4> {
    typedef RawF4 Raw;
    static __device__ __forceinline__ Raw load(const uint8_t *data, const uint8_t *scales, int64_t row_bytes,
                                               int64_t r, int b, int c, int) {
        return load_f4(data + r * row_bytes + (int64_t)b * 128, scales + r * (row_bytes / 8) + (int64_t)b * 16, c);
    }
};

template <>
struct Loader<T_FP8> {
    typedef RawF8 Raw;
    static __device__ __forceinline__ Raw load(const uint8_t *data, const uint8_t *scales, int64_t row_bytes,
                                               int64_t r, int b, int c, int) {
        return load_f8(data + r * row_bytes + (int64_t)b * 256, scales + (r >> 7) * (row_bytes / 64), b, c);
    }
};

}  // namespace qg
