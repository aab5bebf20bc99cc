// Launch arguments of the row-invariant MFMA product (kernels in qg_mma.hpp),
// shared by the host dispatcher and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// Weight superblocks each wave keeps in flight (a ring refills behind the
// computation when a wave has more).
constexpr int kMmaDepth = 3;
// Decode path: staging rounds of two 32-byte x items per lane, at most.
constexpr int kMmaDecRounds = 4;

struct MSeg {
    const uint8_t *data;     // superblocks, or NVFP4 codes
    const uint8_t *scales;   // NVFP4 e4m3 scales or FP8 bf16 block scales, else null
    float *y;                // [n][m]
    const float *resid;      // [n][m] or null
    const uint8_t *data2;    // SwiGLU's up matrix (same shape and type as the gate); else null
    const uint8_t *scales2;  // its scales
    float *y2;               // unused
    int64_t row_bytes;       // bytes per stored row (NVFP4, FP8: codes)
    int32_t type;
    int32_t m;
    int32_t ks;              // K phases per row tile (1, 2, 4, 8 or 16): phase p sums superblocks
                             // p, p + ks, ...; the phases' partials are added in phase order.
                             // A function of (type, m, k) only.
    int32_t wg_begin;        // first workgroup of this matrix
    int32_t dec;             // 1: every wave stages its own x (decode path, np = 1; needs
                             //    ceil(nb/ks) <= kMmaDepth (2 with two tiles per wave),
                             //    16*n*ceil(nb/ks) <= 128*kMmaDecRounds, and LDS for
                             //    wv*ceil(nb/ks)*n*576 bytes after the 144 of zeros)
    int32_t tiled;           // K-quants: 16-row tiled layout (qg_weight.layout = QG_LAYOUT_TILES)
};

struct MmaArgs {
    MSeg seg[3];
    const void *x;           // fp16 [n][k]
    int32_t nseg;
    int32_t k;
    int32_t nb;              // k / 256
    int32_t n;               // tokens, 1..32
    int32_t kc;              // superblocks per staged x chunk
    int32_t wv;              // waves per workgroup (4, 8, 10 or 16; 8 or 16 when np > 1 or for SwiGLU,
                             // 10 only with np = 2 in plain launches)
    int32_t nt;              // weight tiles per wave (1)
    int32_t mode;            // MODE_PLAIN or MODE_SWIGLU
    int32_t np;              // phases per wave (1, 2 or 4; divides every segment's ks): a row
                             // tile has kw = ks / np waves, wave w holding phases w, w + kw, ...
    int32_t xch;             // SwiGLU: 16-byte LDS unit where the gate sums are handed over
    uint32_t nmagic;         // n >= 2: floor(2^32 / n) + 1, so r / n = umulhi(r, nmagic) for r < 2^16
};

// ts: bit set of the weight types in the launch (TS_Q4 | ...); grid: workgroups of
// 64 * A.wv threads; lds: dynamic LDS bytes.  np > 1 and SwiGLU take one weight type
// per launch and workgroups of 8 or 16 waves.
hipError_t launch_mma(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st);
hipError_t launch_mma_w4(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st);
hipError_t launch_mma_w8(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st);
hipError_t launch_mma_w16(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st);
hipError_t launch_mma_w10(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st);   // np = 2, plain

}  // namespace qg
