// Calibration kernels: a plain streaming read of a contiguous buffer, the reference
// the gather kernels' bandwidth is read against on the same GPU (and a kernel of
// known traffic for scaling hardware byte counters); and a bare replay of a recorded
// list of row addresses, the rate the same access pattern reaches without any
// address computation or arithmetic.
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

// Replay of a recorded gather: workgroup i (four wavefronts) reads, for each j < counts[i],
// the row of RB bytes at base + offsets[i * max_keys + j] and the one plane_delta bytes
// further, with the row-contiguous 16-byte loads of the gather kernels (LPR lanes per
// row, 64 / LPR rows per wave instruction, four instructions per plane and batch, marked
// non-temporal like the decode kernel's row loads) and two batches in flight per
// wavefront. Keys are dealt to the wavefronts in batches.
// A row whose bytes (either plane) would leave [base, base + region) is skipped.
template <int RB>
__global__ void __launch_bounds__(256) gather_replay_kernel(const char *base, uint64_t region, const int64_t *offsets,
                                                            const int32_t *counts, uint32_t max_keys,
                                                            int64_t plane_delta, uint32_t *sink)
{
    constexpr int LPR = RB / 16;                 // lanes per row
    constexpr int RPI = 64 / LPR;                // rows per wave instruction
    constexpr int NR = 4 * RPI;                  // rows per wavefront and batch
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t item = blockIdx.x;
    int n = counts[item];
    n = n < 0 ? 0 : (n > (int)max_keys ? (int)max_keys : n);
    const int64_t *my = offsets + item * max_keys;
    const int row = lane / LPR, chunk = lane % LPR;
    const int nb = (n + 4 * NR - 1) / (4 * NR);  // batches of the four wavefronts together
    u32x4 acc = {0u, 0u, 0u, 0u};
    u32x4 k[2][4], v[2][4];
    bool ok[2][4];
    // every load is issued (a key past the count or out of the region reads the first
    // row of the region and is not folded): loads under a branch would make the
    // compiler drain the memory counter at each join
    auto issue = [&](int t, int slot) {
        int64_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = t * 4 * NR + w * NR + i * RPI + row;
            o[i] = my[j < n ? j : n - 1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = t * 4 * NR + w * NR + i * RPI + row;
            const bool in = j < n && o[i] >= 0 && (uint64_t)o[i] + RB <= region && o[i] + plane_delta >= 0 &&
                            (uint64_t)(o[i] + plane_delta) + RB <= region;
            ok[slot][i] = in;
            const char *kr = in ? base + o[i] : base;
            const char *vr = in ? base + o[i] + plane_delta : base;
            k[slot][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kr + chunk * 16));
            v[slot][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vr + chunk * 16));
        }
    };
    if (nb > 0)
        issue(0, 0);
    if (nb > 1)
        issue(1, 1);
    for (int t = 0; t < nb; t += 2) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (t + s < nb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4 x = k[s][i] ^ v[s][i];
                    acc ^= ok[s][i] ? x : u32x4{0u, 0u, 0u, 0u};
                }
                if (t + s + 2 < nb)
                    issue(t + s + 2, s);
            }
        }
    }
    sink[item * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

int launch_gather_replay(const void *base, uint64_t region, const int64_t *offsets, const int32_t *counts,
                         uint32_t items, uint32_t max_keys, uint32_t row_bytes, int64_t plane_delta, uint32_t *sink,
                         void *stream)
{
    if (items == 0)
        return 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const char *b = static_cast<const char *>(base);
    switch (row_bytes) {
    case 64: hipLaunchKernelGGL(gather_replay_kernel<64>, dim3(items), dim3(256), 0, st, b, region, offsets, counts, max_keys, plane_delta, sink); break;
    case 128: hipLaunchKernelGGL(gather_replay_kernel<128>, dim3(items), dim3(256), 0, st, b, region, offsets, counts, max_keys, plane_delta, sink); break;
    case 256: hipLaunchKernelGGL(gather_replay_kernel<256>, dim3(items), dim3(256), 0, st, b, region, offsets, counts, max_keys, plane_delta, sink); break;
    case 512: hipLaunchKernelGGL(gather_replay_kernel<512>, dim3(items), dim3(256), 0, st, b, region, offsets, counts, max_keys, plane_delta, sink); break;
    case 1024: hipLaunchKernelGGL(gather_replay_kernel<1024>, dim3(items), dim3(256), 0, st, b, region, offsets, counts, max_keys, plane_delta, sink); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

int launch_stream_read(const void *src, uint64_t bytes, void *sink, uint32_t grid, void *stream)
{
    if (grid == 0)
        return 0;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kStreamThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), bytes / 16, static_cast<uint32_t *>(sink));
    return (int)hipGetLastError();
}

}  // namespace qsa
