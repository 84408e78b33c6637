// kivi_probe.hip -- measurement helper (not a step of the method): a plain streaming read.
//
// Reads a device buffer once, 16 bytes per lane per load, in a grid-stride sweep that keeps the
// whole chip's reads on one contiguous front, four independent loads in flight per lane, one
// 16-wave workgroup per CU.  Of the read patterns measured on MI355X (grid-stride with 256 to
// 8,192 workgroups of 256 to 1,024 threads and 2 to 8 loads in flight, contiguous per-workgroup
// chunks, non-temporal loads), this one read fastest at 403 MB and 1 GiB: 6.0-6.2 TB/s.  It gives the read ceiling that the decode kernels
// are set against, and, run untimed over a buffer larger than the 256 MB Infinity Cache, it
// evicts a working set from it between timed launches.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_internal.h"

namespace kivi {

constexpr int kProbeBlock = 1024;

__global__ __launch_bounds__(kProbeBlock) void read_probe_kernel(const uint4* src, size_t n, uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * kProbeBlock;
    size_t i = (size_t)blockIdx.x * kProbeBlock + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // one word per workgroup, so the loads are not dropped
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc ^= __shfl_xor(acc, m, 64);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t s, hipEvent_t t0,
                             hipEvent_t t1) {
    const size_t n = bytes / 16;
    hipExtLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeBlock), 0, s, t0, t1, 0,
                          static_cast<const uint4*>(src), n, sink);
    return hipGetLastError();
}

}  // namespace kivi
