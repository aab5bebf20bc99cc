// Row-invariant MFMA product, workgroups of 4 waves.
#include "qg_mma_inst.hpp"

namespace qg {
hipError_t launch_mma_w4(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    return launch_wv<4>(A, ts, grid, lds, st);
}
}  // namespace qg
