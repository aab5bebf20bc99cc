// Dispatch of the row-invariant MFMA product by workgroup size (qg_mma_w*.hip).
#include "qg_mma_launch.h"

namespace qg {

hipError_t launch_mma(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    switch (A.wv) {
    case 4: return launch_mma_w4(A, ts, grid, lds, st);
    case 8: return launch_mma_w8(A, ts, grid, lds, st);
    case 10: return launch_mma_w10(A, ts, grid, lds, st);
    case 16: return launch_mma_w16(A, ts, grid, lds, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qg
