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

// bm x bn tile per workgroup: (128, 128), (128, 64) or (64, 64).
hipError_t launch_prefill(const PrefillArgs &a, int bm, int bn, hipStream_t st);

}  // namespace qg
