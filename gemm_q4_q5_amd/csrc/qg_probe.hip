// Read-stream probe (gfx950): the HBM rate of a plain 16-byte-load stream over
// the same bytes a weight product reads, with no arithmetic on them.  The XOR of
// every 32-bit word is folded into *out so that no load can be dropped.
#include <algorithm>

#include "qg_kernels.h"

namespace qg {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 2;   // independent 16-byte loads in flight per thread

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(ReadArgs A) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    for (int r = 0; r < A.nreg; ++r) {   // uniform
        const uint4 *p = A.p[r];
        const int64_t n = A.n16[r];
        int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
        for (; i + (kReadUnroll - 1) * stride < n; i += kReadUnroll * stride) {
            uint4 v[kReadUnroll];
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
            for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
        for (; i < n; i += stride) {
            const uint4 v = p[i];
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    __shared__ uint32_t wx[kReadThreads / 64];
    if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = 0;
#pragma unroll
        for (int w = 0; w < kReadThreads / 64; ++w) v ^= wx[w];
        // one vector atomic per workgroup, spread over slots a cache line apart
        // (atomics on one address serialize in L2)
        atomicXor(A.out + (blockIdx.x % kReadSlots) * kReadSlotStride, v);
    }
}

hipError_t launch_stream_read(const ReadArgs &A, hipStream_t st) {
    int64_t total = 0;
    for (int r = 0; r < A.nreg; ++r) total += A.n16[r];
    const int64_t want = (total + kReadThreads * kReadUnroll - 1) / (kReadThreads * kReadUnroll);
    // up to 16 workgroups per CU, grid-stride beyond (a sweep of 1..32 per CU and
    // 1..8 loads per thread over a 28 MB cold stream moved the time by under 10 %)
    const int grid = (int)std::min<int64_t>(std::max<int64_t>(want, 1), 256 * 16);
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, st, A);
    return hipGetLastError();
}

}  // namespace qg
