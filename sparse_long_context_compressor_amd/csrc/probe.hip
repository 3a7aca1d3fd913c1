// probe.hip -- a streaming HBM read used to measure the GPU's practical read
// bandwidth beside the published peak: every 16-byte unit of a buffer is read
// once (grid-stride, four loads in flight per thread) and folded into one
// word per workgroup, so that no load can be dropped.

#include "slc_internal.hpp"

namespace slc {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, int64_t units,
                                                          uint32_t *sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    int64_t u = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    for (; u + 3 * stride < units; u += 4 * stride) {
        const u32x4 a = buf[u], b = buf[u + stride], c = buf[u + 2 * stride], d = buf[u + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; u < units; u += stride) acc ^= buf[u];
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __shared__ uint32_t part[256];
    part[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < 256; i++) r ^= part[i];
        sink[blockIdx.x] = r;
    }
}

hipError_t launch_stream_read(const void *buf, int64_t units, uint32_t *sink, int blocks,
                              hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(buf), units, sink);
    return hipGetLastError();
}

}  // namespace slc
