// Read-stream probe (gfx950): the HBM rate of a plain 16-byte-load stream over
// the same bytes a weight product reads, with no arithmetic on them.  The XOR of
// every 32-bit word is folded into *out so that no load can be dropped.
#include "qg_kernels.h"

namespace qg {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;   // independent 16-byte loads in flight per thread
constexpr int64_t kReadTile = (int64_t)kReadThreads * kReadUnroll;   // 16-byte units per workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b reads one contiguous tile of 16 KB (the regions' tiles one after
// another), four non-temporal 16-byte loads per thread, all issued before any is
// used.  Measured on cold graph-launched streams of 6 to 219 MB, this shape (one
// tile per workgroup, non-temporal loads) beat grid-stride loops with 2 to 16 loads
// in flight per thread by 5 to 15 %.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(ReadArgs A) {
    int64_t t = blockIdx.x;
    int r = 0;
    while (r + 1 < A.nreg && t >= (A.n16[r] + kReadTile - 1) / kReadTile) {   // uniform
        t -= (A.n16[r] + kReadTile - 1) / kReadTile;
        ++r;
    }
    const u32x4 *p = reinterpret_cast<const u32x4 *>(A.p[r]);
    const int64_t n = A.n16[r], base = t * kReadTile + threadIdx.x;
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kReadThreads;
        v[u] = i < n ? __builtin_nontemporal_load(p + i) : (u32x4){0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    __shared__ uint32_t wx[kReadThreads / 64];
    if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
#pragma unroll
        for (int w = 0; w < kReadThreads / 64; ++w) x ^= wx[w];
        // one vector atomic per workgroup, spread over slots a cache line apart
        // (atomics on one address serialize in L2)
        atomicXor(A.out + (blockIdx.x % kReadSlots) * kReadSlotStride, x);
    }
}

hipError_t launch_stream_read(const ReadArgs &A, hipStream_t st) {
    int64_t tiles = 0;
    for (int r = 0; r < A.nreg; ++r) tiles += (A.n16[r] + kReadTile - 1) / kReadTile;
    if (tiles < 1 || tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)tiles), dim3(kReadThreads), 0, st, A);
    return hipGetLastError();
}

}  // namespace qg
