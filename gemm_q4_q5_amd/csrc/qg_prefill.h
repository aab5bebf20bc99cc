// Launch arguments of the prefill-chunk GEMM.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

struct PrefillArgs {
    const uint8_t *data;     // weight rows (superblocks or NVFP4 codes)
    const uint8_t *scales;   // NVFP4 e4m3 scales, else null
    const void *x;           // fp16 [n][k]
    float *y;                // fp32 [n][m]
    int64_t row_bytes;
    int64_t m, n;
    int32_t k;
    int32_t type;
    int32_t tiled;           // K-quants: 16-row tiles (qg_weight.layout = QG_LAYOUT_TILES)
    int32_t pad;
};

// The unit of the call's size limit: blocks of 64 tokens x 64 weight rows (the
// workgroups take 64 x 128, or 64 x 80 for Q6_K in two K halves, so fewer of them).
constexpr int kPrefillBlockM = 64, kPrefillBlockN = 64;
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st);

}  // namespace qg
