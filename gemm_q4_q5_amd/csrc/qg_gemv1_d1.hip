// Single-token kernels whose lanes hold 1 superblock slot each, one
// instantiation per weight-type set (a launch carries only the register
// footprint of the types it streams).
#include "qg_gemv.hpp"

namespace qg {

hipError_t launch_gemv1_d1(const GemvArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    return launch_gemv1_d<1>(A, ts, grid, lds, st);
}

}  // namespace qg
