// probe.hip -- streaming-read probe: the HBM read rate a kernel that only
// reads can reach on this device, the ceiling the memory-bound kernels of
// the library are compared with ("3.6 Quantization": batch-1 decode time is
// the bytes read over the memory bandwidth).
//
// 1024 workgroups of 256 lanes walk the buffer grid-stride, two 16-byte
// non-temporal loads per lane per step (the shape that read fastest across
// 34 MB .. 1 GB buffers on MI355X); the words are xor-folded so the loads
// are live, and a lane stores only if its fold equals a value the caller
// never expects, so the sink is in practice never written.
#include "common.hpp"
#include "launch.hpp"

namespace lq {

namespace {

constexpr int kProbeGrid = 1024;
constexpr int kProbeUnroll = 2;

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *__restrict__ p, int64_t n16,
                                                          uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256 * kProbeUnroll;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 * kProbeUnroll + threadIdx.x; i < n16; i += stride) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t j = i + u * 256;
            v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

int64_t read_probe_sink_words() { return kProbeGrid; }

hipError_t launch_read_probe(const void *p, int64_t bytes, uint32_t *sink, hipStream_t st) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeGrid), dim3(256), 0, st, static_cast<const u32x4 *>(p), bytes / 16,
                       sink);
    return hipGetLastError();
}

}  // namespace lq
