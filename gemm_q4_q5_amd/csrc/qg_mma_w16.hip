// Row-invariant MFMA product, workgroups of 16 waves.
#include "qg_mma_inst.hpp"

namespace qg {
hipError_t launch_mma_w16(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    return launch_wv<16>(A, ts, grid, lds, st);
}
}  // namespace qg
