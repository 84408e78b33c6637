// kivi_probe.hip -- measurement helper (not a step of the method): a streaming read.
//
// Reads a device buffer once, 16 bytes per lane per load, in a grid-stride sweep that keeps the
// whole chip's reads on one contiguous front, four independent loads in flight per lane, one
// 16-wave workgroup per CU.  With plain loads it reads 403 MB in 64.6-64.9 us (6.2 TB/s) and
// 1 GiB in 174 us; with non-temporal loads (the streaming form) 58.4-58.8 us (6.9 TB/s, 0.86 of
// the HBM peak) and 159 us.  The streaming form gives the read ceiling the decode kernels are set
// against; the plain form, run untimed over a buffer larger than the 256 MB Infinity Cache,
// evicts a working set from it between timed launches (plain loads allocate in that cache).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

constexpr int kProbeBlock = 1024;

template <bool STREAM>
__global__ __launch_bounds__(kProbeBlock) void read_probe_kernel(const uint4* src, size_t n, uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * kProbeBlock;
    size_t i = (size_t)blockIdx.x * kProbeBlock + threadIdx.x;
    auto ld = [&](size_t k) { return STREAM ? stream_load16(src + k) : src[k]; };
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        const uint4 a = ld(i), b = ld(i + stride), c = ld(i + 2 * stride), d = ld(i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n; i += stride) {
        const uint4 a = ld(i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // one word per workgroup, so the loads are not dropped
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc ^= __shfl_xor(acc, m, 64);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, bool streaming, hipStream_t s,
                             hipEvent_t t0, hipEvent_t t1) {
    const size_t n = bytes / 16;
    if (streaming)
        hipExtLaunchKernelGGL(read_probe_kernel<true>, dim3(kProbeBlocks), dim3(kProbeBlock), 0, s, t0, t1, 0,
                              static_cast<const uint4*>(src), n, sink);
    else
        hipExtLaunchKernelGGL(read_probe_kernel<false>, dim3(kProbeBlocks), dim3(kProbeBlock), 0, s, t0, t1, 0,
                              static_cast<const uint4*>(src), n, sink);
    return hipGetLastError();
}

}  // namespace kivi
