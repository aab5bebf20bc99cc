// Row-invariant MFMA product, workgroups of 10 waves: five row tiles of two phases
// each (a K split in four phases), for the plain several-token launches whose grid
// of one such workgroup per CU covers more CUs than 8- or 16-wave workgroups do
// (the 9728-row gate/up pair: 244 workgroups against 152).
#include "qg_mma_inst.hpp"

namespace qg {
hipError_t launch_mma_w10(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    if (A.np != 2 || A.mode != MODE_PLAIN || A.nt != 1) return hipErrorInvalidValue;
    return A.n > 16 ? launch_ts<2, 10, 1, false, 2>(A, ts, grid, lds, st)
                    : launch_ts<1, 10, 1, false, 2>(A, ts, grid, lds, st);
}
}  // namespace qg
