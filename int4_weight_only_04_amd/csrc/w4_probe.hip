// A kernel that only reads: the practical ceiling against which the GEMVs'
// bandwidth is judged.  It streams a buffer with the same 16-byte
// non-temporal loads as the GEMV's weight stream (each thread issues its 8
// loads before combining them), and stores the XOR of every word a
// workgroup read (2048 x 16 bytes per workgroup) into word blockIdx % 1024 of
// `sink`, so the loads cannot be dropped.  Timing launches of it with the
// sizes of a sweep's matrices, one per matrix and in the same order, gives
// the time a sweep of pure reads with the same kernel boundaries takes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4_internal.h"

namespace w4i {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const probe_u32x4* __restrict__ src, int64_t n16,
                                                                   uint32_t* __restrict__ sink)
{
    const int64_t base = (int64_t)blockIdx.x * (kProbeThreads * kProbeUnroll) + threadIdx.x;
    probe_u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
        const int64_t i = base + (int64_t)u * kProbeThreads;
        v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : probe_u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    // the XOR of every word the workgroup read, into word blockIdx.x % 1024
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
    __shared__ uint32_t part[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = part[0];
#pragma unroll
        for (int w = 1; w < kProbeThreads / 64; ++w) t ^= part[w];
        sink[blockIdx.x % kProbeSinkWords] = t;
    }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream)
{
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t per = (int64_t)kProbeThreads * kProbeUnroll;
    const int64_t grid = (n16 + per - 1) / per;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const probe_u32x4*>(buf), n16, sink);
    return hipGetLastError();
}

}  // namespace w4i
