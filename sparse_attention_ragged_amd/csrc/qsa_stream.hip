// Calibration kernel: a plain streaming read of a contiguous buffer, the reference
// the gather kernels' bandwidth is read against on the same GPU (and a kernel of
// known traffic for scaling hardware byte counters).
//
// Every byte of [src, src + bytes) is loaded exactly once with 16-byte loads, four
// per thread in flight per step, consecutive lanes on consecutive 16-byte chunks
// (each wavefront instruction covers 1 KiB). The loaded words are folded into one
// xor per workgroup and written to sink[blockIdx.x], so the loads cannot be removed.
#include "qsa_device.hpp"

namespace qsa {

namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const u32x4 *src, uint64_t chunks,
                                                                    uint32_t *sink)
{
    const uint64_t stride = (uint64_t)gridDim.x * kStreamThreads;
    uint64_t i = (uint64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kStreamUnroll - 1) * stride < chunks; i += kStreamUnroll * stride) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u)
            acc ^= v[u];
    }
    for (; i < chunks; i += stride)
        acc ^= __builtin_nontemporal_load(src + i);
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int off = 32; off > 0; off >>= 1)
        x ^= (uint32_t)__shfl_xor((int)x, off);
    __shared__ uint32_t part[kStreamThreads / 64];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
        for (int w = 0; w < kStreamThreads / 64; ++w)
            y ^= part[w];
        sink[blockIdx.x] = y;
    }
}

}  // namespace

int launch_stream_read(const void *src, uint64_t bytes, void *sink, uint32_t grid, void *stream)
{
    if (grid == 0)
        return 0;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), bytes / 16, static_cast<uint32_t *>(sink));
    return (int)hipGetLastError();
}

}  // namespace qsa
