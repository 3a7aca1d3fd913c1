// bench_probe.hip -- measurement only, not part of the library: a streaming
// HBM read that gives the benchmark the GPU's practical read bandwidth beside
// the published peak.  Every 16-byte unit of a buffer is read exactly once
// (one contiguous region per workgroup, eight independent non-temporal loads
// in flight per thread) and folded into one word per workgroup, so that no load can
// be dropped.  Built by
// bench.py's build_probe() into bench_probe.so, loaded by bench.py only.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *buf, int64_t units,
                                                          uint32_t *sink) {
    constexpr int kInFlight = 8;
    // workgroup b reads one contiguous region, units [b per, (b + 1) per)
    const int64_t per = (units + gridDim.x - 1) / gridDim.x;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t hi = lo + per < units ? lo + per : units;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t u = lo + threadIdx.x;
    for (; u + (kInFlight - 1) * 256 < hi; u += kInFlight * 256) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int i = 0; i < kInFlight; i++) v[i] = __builtin_nontemporal_load(buf + u + i * 256);
#pragma unroll
        for (int i = 0; i < kInFlight; i++) acc ^= v[i];
    }
    for (; u < hi; u += 256) acc ^= __builtin_nontemporal_load(buf + u);
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

// 0: launched; 1: bad arguments (nothing launched); 2: launch failure.
extern "C" int bench_stream_read(const void *buf, size_t bytes, uint32_t *sink, int blocks,
                                 void *stream) {
    if (!buf || !sink || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0 ||
        blocks < 1 || blocks > 65536)
        return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf),
                       static_cast<int64_t>(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
