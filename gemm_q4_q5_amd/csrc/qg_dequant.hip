// Dequant probe (gfx950): writes every weight of a matrix as fp32 through the
// same loads and decoders the products use.
#include "qg_loads.hpp"

namespace qg {

// thread (r, b, c) writes the 64 weights of chunk c of block b.
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs A) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = A.m * (int64_t)A.nb * 4;
    if (gid >= total) return;
    const int c = (int)(gid & 3);
    const int64_t b = (gid >> 2) % A.nb;
    const int64_t r = (gid >> 2) / A.nb;
    float *out = A.out + r * (int64_t)A.k + b * 256;
    if (A.type == T_Q4_K || A.type == T_Q5_K) {
        const bool q5 = A.type == T_Q5_K;
        const RawKq R = q5 ? Loader<T_Q5_K>::load(A.data, A.scales, A.row_bytes, r, (int)b, c, A.tiled)
                           : Loader<T_Q4_K>::load(A.data, A.scales, A.row_bytes, r, (int)b, c, A.tiled);
        const KqCoef cf = kq_coef(R.hdr, kq_lane_consts(c));
        const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
        const uint32_t hw[8] = {R.h0.x, R.h0.y, R.h0.z, R.h0.w, R.h1.x, R.h1.y, R.h1.z, R.h1.w};
        for (int i = 0; i < 8; ++i) {
            const Quad qd = q5 ? q5_quad(qw[i], pair_bytes(hw[i], hw[i], kSelAligned) >> (2 * c))
                               : q4_quad(qw[i]);
            const uint32_t lo[2] = {qd.lo01, qd.lo23}, hi[2] = {qd.hi01, qd.hi23};
            for (int e = 0; e < 2; ++e) {
                const int pos = 4 * i + 2 * e;
                out[64 * c + pos] = __builtin_fmaf(cf.a0, f16lo(lo[e]) - 1024.0f, cf.b0);
                out[64 * c + pos + 1] = __builtin_fmaf(cf.a0, f16hi(lo[e]) - 1024.0f, cf.b0);
                out[64 * c + 32 + pos] = __builtin_fmaf(cf.a1, f16lo(hi[e]) - 256.0f, cf.b1);
                out[64 * c + 32 + pos + 1] = __builtin_fmaf(cf.a1, f16hi(hi[e]) - 256.0f, cf.b1);
            }
        }
    } else if (A.type == T_Q6_K) {
        const RawQ6 R = Loader<T_Q6_K>::load(A.data, A.scales, A.row_bytes, r, (int)b, c, A.tiled);
        const int s = c >> 1, h = c & 1;
        const uint32_t sel = R.mis ? kSelMis : kSelAligned;
        const uint32_t av[5] = {R.a.x, R.a.y, R.a.z, R.a.w, R.a4};
        const uint32_t bv[5] = {R.b.x, R.b.y, R.b.z, R.b.w, R.b4};
        const uint32_t hv[5] = {R.h.x, R.h.y, R.h.z, R.h.w, R.h4};
        const uint32_t l0 = __builtin_amdgcn_alignbyte(R.s01.y, R.s01.x, R.mis);
        const uint32_t l1 = __builtin_amdgcn_alignbyte(R.s2, R.s01.y, R.mis);
        float coef[4];
        q6_coefs(l0, l1, f16lo(R.d), h, coef);
        for (int i = 0; i < 4; ++i) {
            const Q6Oct o = q6_oct(pair_bytes(av[i + 1], av[i], sel), pair_bytes(bv[i + 1], bv[i], sel),
                                   pair_bytes(hv[i + 1], hv[i], sel));
            for (int g = 0; g < 4; ++g) {
                const int pos = 128 * s + 32 * g + 16 * h + 4 * i;
                // coef[g] * (v - bias) = d * sc * (q - 32), every step exact.
                const float bias = g < 2 ? 1056.0f : 384.0f;
                out[pos] = coef[g] * (f16lo(o.v[g][0]) - bias);
                out[pos + 1] = coef[g] * (f16hi(o.v[g][0]) - bias);
                out[pos + 2] = coef[g] * (f16lo(o.v[g][1]) - bias);
                out[pos + 3] = coef[g] * (f16hi(o.v[g][1]) - bias);
            }
        }
    } else if (A.type == T_FP8) {
        const RawF8 R = Loader<T_FP8>::load(A.data, A.scales, A.row_bytes, r, (int)b, c, 0);
        const float sc = bf16_lo(R.sc);
        const uint32_t qw[16] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w,
                                 R.q2.x, R.q2.y, R.q2.z, R.q2.w, R.q3.x, R.q3.y, R.q3.z, R.q3.w};
        for (int i = 0; i < 16; ++i)
            for (int e = 0; e < 4; ++e) out[64 * c + 4 * i + e] = e4m3_at(qw[i], e) * sc;   // exact
    } else {
        const RawF4 R = load_f4(A.data + r * A.row_bytes + b * 128,
                                A.scales + r * (A.row_bytes / 8) + b * 16, c);
        const uint32_t qw[8] = {R.q0.x, R.q0.y, R.q0.z, R.q0.w, R.q1.x, R.q1.y, R.q1.z, R.q1.w};
        for (int i = 0; i < 8; ++i) {
            const float sc = e4m3_at(R.sc, i >> 1);
            for (int j = 0; j < 4; ++j) {
                const uint32_t v = fp4_pair(qw[i], j);
                out[64 * c + 8 * i + 2 * j] = sc * f16lo(v);
                out[64 * c + 8 * i + 2 * j + 1] = sc * f16hi(v);
            }
        }
    }
}

// Row-major superblocks -> the 16-row tiled layout (tile_chunk, tile_src): thread o
// writes 16-bit unit o of the tiled copy (every offset is even); rows past m in the
// last tile repeat row m-1.
__global__ __launch_bounds__(256) void pack_tiles_kernel(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                                        int64_t m, int64_t row_bytes, int sbytes, int64_t units) {
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= units) return;
    const int64_t half = 8 * (int64_t)sbytes, nb = row_bytes / sbytes;   // 16-bit units per chunk
    const int e = (int)(o % half) * 2;                                     // byte of the chunk
    const int64_t ch = o / half;                                           // chunk (tile, superblock)
    const int64_t b = ch % nb, t = ch / nb;
    int j = 0;
    const int off = tile_src(sbytes, e, j);
    const int64_t r = t * 16 + j < m ? t * 16 + j : m - 1;
    dst[o] = src[(r * row_bytes + b * sbytes + off) / 2];
}

hipError_t launch_pack_tiles(const uint8_t *src, uint8_t *dst, int64_t m, int64_t row_bytes, int sbytes,
                             hipStream_t st) {
    const int64_t units = (m + 15) / 16 * 16 * row_bytes / 2;
    hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t *>(src), reinterpret_cast<uint16_t *>(dst), m, row_bytes,
                       sbytes, units);
    return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs &A, hipStream_t st) {
    const int64_t total = A.m * (int64_t)A.nb * 4;
    const int64_t grid = (total + 255) / 256;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)grid), dim3(256), 0, st, A);
    return hipGetLastError();
}

}  // namespace qg
