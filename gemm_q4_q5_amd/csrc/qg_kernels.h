// Launch-argument structures shared by the host dispatcher and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

enum : int { MODE_PLAIN = 0, MODE_SWIGLU = 1 };

// Weight-type sets a kernel instantiation handles.
enum : int { TS_Q4 = 1, TS_Q5 = 2, TS_Q6 = 4, TS_F4 = 8, TS_F8 = 16, TS_ALL = 31 };

constexpr __host__ __device__ int type_bit(int type) {
    return type == 12 ? TS_Q4 : type == 13 ? TS_Q5 : type == 14 ? TS_Q6 : type == 1001 ? TS_F4 : TS_F8;
}

struct DequantArgs {
    const uint8_t *data;
    const uint8_t *scales;
    float *out;
    int64_t row_bytes;
    int64_t m;
    int32_t k;
    int32_t nb;
    int32_t type;
    int32_t tiled;   // K-quants: 16-row tiles (qg_weight.layout = QG_LAYOUT_TILES)
};

hipError_t launch_dequant(const DequantArgs &a, hipStream_t st);
// Copy of a row-major K-quant matrix in 16-row tiles (16 * ceil(m/16) rows; the rows
// past m repeat row m-1).
hipError_t launch_pack_tiles(const uint8_t *src, uint8_t *dst, int64_t m, int64_t row_bytes, int sbytes,
                             hipStream_t st);

constexpr int kReadMaxRegions = 3;
constexpr int kReadSlots = 64;         // XOR accumulators of the read probe ...
constexpr int kReadSlotStride = 32;    // ... one per 128-byte line: out is 2048 words

struct ReadArgs {
    const uint4 *p[kReadMaxRegions];
    int64_t n16[kReadMaxRegions];   // 16-byte units per region
    uint32_t *out;
    int32_t nreg;
    int32_t pad;
};

hipError_t launch_stream_read(const ReadArgs &a, hipStream_t st);

}  // namespace qg
