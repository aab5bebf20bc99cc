// Instantiations of the row-invariant MFMA product for one workgroup size
// (included by qg_mma_w4.hip, qg_mma_w8.hip and qg_mma_w16.hip).
#pragma once
#include "qg_mma.hpp"

namespace qg {

template <int TS, int NG, int WV, int NT, bool SW, int NP>
static hipError_t launch_one(const MmaArgs &A, int grid, size_t lds, hipStream_t st) {
    const void *fn = (const void *)mma_kernel<TS, NG, WV, NT, SW, NP>;
    if (lds > 65536) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((mma_kernel<TS, NG, WV, NT, SW, NP>), dim3(grid), dim3(64 * WV), lds, st, A);
    return hipGetLastError();
}

template <int NG, int WV, int NT, bool SW, int NP>
static hipError_t launch_ts(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    switch (ts) {
    case TS_Q4: return launch_one<TS_Q4, NG, WV, NT, SW, NP>(A, grid, lds, st);
    case TS_Q5: return launch_one<TS_Q5, NG, WV, NT, SW, NP>(A, grid, lds, st);
    case TS_Q6:
        // Q6_K in 16-wave workgroups with four phases of two token groups does not fit
        // 128 registers; the host never asks for it.
        if constexpr (WV == 16 && NP == 4 && NG == 2) return hipErrorInvalidValue;
        else return launch_one<TS_Q6, NG, WV, NT, SW, NP>(A, grid, lds, st);
    case TS_F4: return launch_one<TS_F4, NG, WV, NT, SW, NP>(A, grid, lds, st);
    case TS_F8: return launch_one<TS_F8, NG, WV, NT, SW, NP>(A, grid, lds, st);
    default:
        // SwiGLU pairs share one type; several phases per wave take one type per launch.
        if constexpr (SW || NP > 1) return hipErrorInvalidValue;
        else if (ts == (TS_Q4 | TS_Q6)) return launch_one<TS_Q4 | TS_Q6, NG, WV, NT, false, 1>(A, grid, lds, st);
        else return launch_one<TS_ALL, NG, WV, NT, false, 1>(A, grid, lds, st);
    }
}

template <int NG, int WV, int NP>
static hipError_t launch_nt(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    if (A.nt != 1) return hipErrorInvalidValue;
    if (A.mode == MODE_SWIGLU) {   // gate and up tile groups in pairs
        if constexpr (WV >= 8) return launch_ts<NG, WV, 1, true, NP>(A, ts, grid, lds, st);
        else return hipErrorInvalidValue;
    }
    return launch_ts<NG, WV, 1, false, NP>(A, ts, grid, lds, st);
}

template <int WV, int NP>
static hipError_t launch_np(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    return A.n > 16 ? launch_nt<2, WV, NP>(A, ts, grid, lds, st) : launch_nt<1, WV, NP>(A, ts, grid, lds, st);
}

template <int WV>
static hipError_t launch_wv(const MmaArgs &A, int ts, int grid, size_t lds, hipStream_t st) {
    if (A.np == 1) return launch_np<WV, 1>(A, ts, grid, lds, st);
    if constexpr (WV >= 8) {
        if (A.np == 2) return launch_np<WV, 2>(A, ts, grid, lds, st);
        if (A.np == 4) return launch_np<WV, 4>(A, ts, grid, lds, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace qg
