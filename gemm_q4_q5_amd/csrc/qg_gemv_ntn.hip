// Multi-token (2..32) instantiations of gemv_kernel, by power-of-two bucket.
#include "qg_gemv.hpp"

namespace qg {

hipError_t launch_gemv_ntn(const GemvArgs &A, int nt, int grid, size_t lds, hipStream_t st) {
    switch (nt) {
    case 2: return launch_one<2, TS_ALL>(A, grid, lds, st);
    case 4: return launch_one<4, TS_ALL>(A, grid, lds, st);
    case 8: return launch_one<8, TS_ALL>(A, grid, lds, st);
    case 16: return launch_one<16, TS_ALL>(A, grid, lds, st);
    case 32: return launch_one<32, TS_ALL>(A, grid, lds, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qg
