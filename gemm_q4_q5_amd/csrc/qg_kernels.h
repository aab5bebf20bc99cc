// Launch-argument structures shared by the host dispatcher and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

enum : int { MODE_PLAIN = 0, MODE_SWIGLU = 1 };

// Weight-type sets a kernel instantiation handles.
enum : int { TS_Q4 = 1, TS_Q5 = 2, TS_Q6 = 4, TS_F4 = 8, TS_ALL = 15 };

constexpr __host__ __device__ int type_bit(int type) {
    return type == 12 ? TS_Q4 : type == 13 ? TS_Q5 : type == 14 ? TS_Q6 : TS_F4;
}

// One weight matrix of a launch (a launch holds up to three sharing x).
struct Seg {
    const uint8_t *data;     // superblocks or NVFP4 codes
    const uint8_t *scales;   // NVFP4 e4m3 scales, else null
    float *y;                // [n][m]
    const float *resid;      // [n][m] or null
    int64_t row_bytes;       // bytes per stored row (NVFP4: codes)
    int32_t type;
    int32_t m;
    int32_t P;               // lanes per row = 4 * P (power of two)
    int32_t lp;              // log2(P)
    int32_t wg_begin;        // first workgroup of this matrix
    int32_t pad;
};

struct GemvArgs {
    Seg seg[3];
    const void *x;           // fp16 [n][k]
    int32_t nseg;
    int32_t k;
    int32_t nb;              // k / 256
    int32_t n;               // tokens
    int32_t kc;              // superblocks per LDS chunk
    int32_t mode;
};

struct DequantArgs {
    const uint8_t *data;
    const uint8_t *scales;
    float *out;
    int64_t row_bytes;
    int64_t m;
    int32_t k;
    int32_t nb;
    int32_t type;
    int32_t pad;
};

// Superblocks one lane loads per round in the single-token kernel; the host
// picks P (lanes per row / 4) so that a lane's share of a row fits one round.
constexpr int kDepth1 = 3;
constexpr int kMaxP = 16;
constexpr int kMaxNb1 = 64;   // superblocks of x the single-token kernel stages at once

hipError_t launch_gemv1_d1(const GemvArgs &a, int ts, int grid, size_t lds, hipStream_t st);
hipError_t launch_gemv1_d2(const GemvArgs &a, int ts, int grid, size_t lds, hipStream_t st);
hipError_t launch_gemv1_d3(const GemvArgs &a, int ts, int grid, size_t lds, hipStream_t st);
hipError_t launch_gemv_ntn(const GemvArgs &a, int nt, int grid, size_t lds, hipStream_t st);
hipError_t launch_dequant(const DequantArgs &a, hipStream_t st);

}  // namespace qg
