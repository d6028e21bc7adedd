// Key compression ("QSACompressKeysPaged": summary, Tensor shapes, execute Parameters
// and Args): sequence b holds key_counts[b] raw index keys (this step's included) at
// positions 0.. of plane 0, kv head 0 of a paged indexer cache. Each complete group of
// `ratio` consecutive keys becomes one block key j (positions j*ratio ..
// j*ratio + ratio - 1): the mean of the group, RMS-normalised over head_dim with the
// weight gamma and eps, then the channel pairs (2i, 2i+1) below rotary_dim turned by
// the rotary table's (cos, sin) pair at the block's first raw position j*ratio. Block
// key j of sequence b is row b * max_blocks + j of block_keys; a trailing partial
// group gives no block key, and rows past a sequence's block count are not written.
//
// HBM-bound streaming: every raw key is read once with 16-byte loads (marked
// non-temporal: measured 4 % faster at the compression workload) and every block key
// written once. A team of TL = head_dim * elem / 16 lanes holds one raw key row,
// one 16-byte chunk per lane (4 fp32 or 8 bf16 channels, so a rotated channel pair
// never straddles two lanes), and computes one block key: it loads the group's rows,
// sums them in fp32, reduces the sum of squares over its lanes with DPP and lane
// shuffles, and writes its chunk of the block key. A workgroup's teams take
// consecutive blocks, so a wavefront's loads cover a few KiB of consecutive positions.
// Ratios 1, 2, 4, 8 and 16 (up to the page size) issue every row load of the block at
// once; other ratios loop over the group four rows at a time. No LDS, no barriers: a
// team whose block does not exist leaves at once.
#include "qsa_device.hpp"
#include "qsa_select_host.hpp"

namespace qsa {
namespace {

// binary32 -> bf16 bits, round to nearest even in integer arithmetic (NaN stays a quiet
// NaN). This kernel measured 5 % faster with it than with the hardware conversion the
// attention kernels use (47 against 49.5 us on the key-compression workload).
__device__ __forceinline__ uint32_t bf16_bits_int(float f)
{
    const uint32_t u = __float_as_uint(f);
    const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t nan = (u >> 16) | 0x40u;
    return (u & 0x7fffffffu) > 0x7f800000u ? nan : rne;
}

template <int DT, int CH>
__device__ __forceinline__ void widen(const u32x4 &v, float *x)
{
    if constexpr (DT == QSA_BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            x[2 * w] = bf16_lo(v[w]);
            x[2 * w + 1] = bf16_hi(v[w]);
        }
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            x[w] = __uint_as_float(v[w]);
    }
}

// The (cos, sin) pair of table row `pos` for channels (ch, ch + 1) as two floats.
__device__ __forceinline__ void rotary_pair(const CompressParams &p, int64_t pos, int ch, float &c, float &s)
{
    const int64_t i = pos * p.rotary_dim + ch;          // even: 4- or 8-byte aligned
    if (p.freq_dtype == QSA_BF16) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(p.freqs) + i);
        c = bf16_lo(w);
        s = bf16_hi(w);
    } else {
        const f32x2_t w = *reinterpret_cast<const f32x2_t *>(static_cast<const float *>(p.freqs) + i);
        c = w[0];
        s = w[1];
    }
}

// Mean, RMS norm, rotation and store of one block key from the fp32 sum of its raw
// rows (acc: this lane's CH channels). Every lane of the team must be here: the sum of
// squares is reduced over the team.
template <int DT, int TL>
__device__ __forceinline__ void finish_block(const CompressParams &p, float (&acc)[16 / Elem<DT>::bytes],
                                             const u32x4 &graw, const float *rc, const float *rs, int64_t b,
                                             int64_t j, int tl, bool write)
{
    constexpr int EB = Elem<DT>::bytes;
    constexpr int CH = 16 / EB;
    const float rf = (float)p.ratio;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        acc[c] = acc[c] / rf;
        ss += acc[c] * acc[c];
    }
    ss = team_sum<TL>(ss);
    const float inv = 1.0f / sqrtf(ss / (float)p.head_dim + p.eps);
    float g[CH];
    widen<DT, CH>(graw, g);
    float y[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
        y[c] = g[c] * acc[c] * inv;
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) {
        const float a = y[2 * i], bb = y[2 * i + 1];
        y[2 * i] = rc[i] * a - rs[i] * bb;
        y[2 * i + 1] = rs[i] * a + rc[i] * bb;
    }
    if (!write)
        return;
    char *dst = static_cast<char *>(p.out) + ((b * p.max_blocks + j) * p.head_dim) * EB + tl * 16;
    u32x4 o;
    if constexpr (DT == QSA_BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            o[w] = bf16_bits_int(y[2 * w]) | (bf16_bits_int(y[2 * w + 1]) << 16);
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            o[w] = __float_as_uint(y[w]);
    }
    *reinterpret_cast<u32x4 *>(dst) = o;
}

// This lane's rotary (cos, sin) pairs for the block starting at raw position pos
// (identity past rotary_dim).
template <int CH>
__device__ __forceinline__ void load_rotary(const CompressParams &p, uint32_t pos, int ch, float *rc, float *rs)
{
#pragma unroll
    for (int i = 0; i < CH / 2; ++i) {
        rc[i] = 1.f;
        rs[i] = 0.f;
        if (ch + 2 * i + 1 < p.rotary_dim)
            rotary_pair(p, pos, ch + 2 * i, rc[i], rs[i]);
    }
}

// Any ratio: one block key per team, the group's rows loaded four at a time.
template <int DT, int TL>
__global__ __launch_bounds__(kCompressThreads) void compress_keys_kernel(CompressParams p)
{
    constexpr int CH = 16 / Elem<DT>::bytes;                  // channels per lane
    constexpr int TPB = kCompressThreads / TL;                // block keys per workgroup
    const int64_t wg_per_seq = (p.blocks_bound + TPB - 1) / TPB;
    const int b = (int)(blockIdx.x / wg_per_seq);
    const int64_t j = (int64_t)(blockIdx.x - (int64_t)b * wg_per_seq) * TPB + threadIdx.x / TL;
    const int tl = threadIdx.x % TL;
    const int32_t kc = p.key_counts[b];
    const int64_t nb = kc > 0 ? kc / p.ratio : 0;
    if (j >= nb || j >= p.blocks_bound)
        return;                                               // whole teams leave together
    const uint32_t pos0 = (uint32_t)(j * p.ratio);            // < 2^31: bounded on the host
    float rc[CH / 2], rs[CH / 2];
    load_rotary<CH>(p, pos0, tl * CH, rc, rs);
    const u32x4 graw = ldg16(static_cast<const char *>(p.gamma) + tl * 16);

    // the group's raw key rows: page-table entry, then the 16-byte chunk of each row;
    // an entry outside the page table or the pool reads a harmless row and drops the block
    float acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
        acc[c] = 0.f;
    bool ok = true;
    const char *base = static_cast<const char *>(p.kv.blocks) + tl * 16;
#pragma unroll 4
    for (int t = 0; t < p.ratio; ++t) {
        bool in_lut, in_pool;
        int32_t slot;
        const uint32_t *e = leaf_entry_ptr(p.kv, b, pos0 + (uint32_t)t, in_lut, slot);
        const uint32_t page = *(in_lut ? e : p.kv.lut);
        const char *row = leaf_row(p.kv, page, slot, 0u, in_pool) + tl * 16;
        ok = ok && in_lut && in_pool;
        const u32x4 v = ldg16_nt(in_lut && in_pool ? row : base);
        float x[CH];
        widen<DT, CH>(v, x);
#pragma unroll
        for (int c = 0; c < CH; ++c)
            acc[c] += x[c];
    }
    finish_block<DT, TL>(p, acc, graw, rc, rs, b, j, tl, ok);
}

// Ratio fixed at compile time (and at most the page size): one block key per team as
// above, but all RATIO row loads of the block are issued at once from the page-table
// entries of its first and last rows (its rows span at most two pages). Measured on
// the indexer workload: as fast as a two-round software pipeline per team and faster
// than several blocks per team, which cost occupancy and serialise the finishing
// work; many short workgroups keep the most row loads in flight.
template <int DT, int TL, int RATIO>
__global__ __launch_bounds__(kCompressThreads) void compress_keys_fixed_kernel(CompressParams p)
{
    constexpr int CH = 16 / Elem<DT>::bytes;
    constexpr int TPB = kCompressThreads / TL;
    const int64_t wg_per_seq = (p.blocks_bound + TPB - 1) / TPB;
    const int b = (int)(blockIdx.x / wg_per_seq);
    const int64_t j = (int64_t)(blockIdx.x - (int64_t)b * wg_per_seq) * TPB + threadIdx.x / TL;
    const int tl = threadIdx.x % TL;
    const int32_t kc = p.key_counts[b];
    const int64_t nb = kc > 0 ? kc / RATIO : 0;
    if (j >= nb || j >= p.blocks_bound)
        return;                                               // whole teams leave together
    const uint32_t pos0 = (uint32_t)(j * RATIO);
    bool in_a, in_b;
    int32_t s_a, s_b;
    const uint32_t *e_a = leaf_entry_ptr(p.kv, b, pos0, in_a, s_a);
    const uint32_t *e_b = leaf_entry_ptr(p.kv, b, pos0 + RATIO - 1, in_b, s_b);
    const uint32_t pg_a = *(in_a ? e_a : p.kv.lut);
    const uint32_t pg_b = *(in_b ? e_b : p.kv.lut);
    float rc[CH / 2], rs[CH / 2];
    load_rotary<CH>(p, pos0, tl * CH, rc, rs);
    const u32x4 graw = ldg16(static_cast<const char *>(p.gamma) + tl * 16);
    const char *base = static_cast<const char *>(p.kv.blocks) + tl * 16;
    u32x4 v[RATIO];
    bool ok = true;
#pragma unroll
    for (int t = 0; t < RATIO; ++t) {
        const bool first = s_a + t < p.kv.page_size;
        const bool in_lut = first ? in_a : in_b;
        bool in_pool;
        const char *row = leaf_row(p.kv, first ? pg_a : pg_b, first ? s_a + t : s_a + t - p.kv.page_size, 0u,
                                   in_pool) + tl * 16;
        ok = ok && in_lut && in_pool;
        v[t] = ldg16_nt(in_lut && in_pool ? row : base);
    }
    float acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
        acc[c] = 0.f;
#pragma unroll
    for (int t = 0; t < RATIO; ++t) {
        float x[CH];
        widen<DT, CH>(v[t], x);
#pragma unroll
        for (int c = 0; c < CH; ++c)
            acc[c] += x[c];
    }
    finish_block<DT, TL>(p, acc, graw, rc, rs, b, j, tl, ok);
}

template <int DT, int TL, int RATIO>
void launch_fixed(const CompressParams &p, hipStream_t s)
{
    const int64_t per_wg = kCompressThreads / TL;
    const dim3 grid((unsigned)((int64_t)p.batch * ((p.blocks_bound + per_wg - 1) / per_wg)));
    hipLaunchKernelGGL((compress_keys_fixed_kernel<DT, TL, RATIO>), grid, dim3(kCompressThreads), 0, s, p);
}

template <int DT, int TL>
int launch_tl(const CompressParams &p, hipStream_t s)
{
    switch (p.kv.page_size >= p.ratio ? p.ratio : 0) {
    case 1: launch_fixed<DT, TL, 1>(p, s); break;
    case 2: launch_fixed<DT, TL, 2>(p, s); break;
    case 4: launch_fixed<DT, TL, 4>(p, s); break;
    case 8: launch_fixed<DT, TL, 8>(p, s); break;
    case 16: launch_fixed<DT, TL, 16>(p, s); break;
    default: {
        constexpr int64_t per_wg = kCompressThreads / TL;
        const dim3 grid((unsigned)((int64_t)p.batch * ((p.blocks_bound + per_wg - 1) / per_wg)));
        hipLaunchKernelGGL((compress_keys_kernel<DT, TL>), grid, dim3(kCompressThreads), 0, s, p);
    }
    }
    return (int)hipGetLastError();
}

template <int DT>
int launch_dt(const CompressParams &p, void *stream)
{
    if (p.batch == 0 || p.blocks_bound == 0)
        return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (compress_team_lanes(Elem<DT>::bytes, p.head_dim)) {
    case 1: return launch_tl<DT, 1>(p, s);
    case 2: return launch_tl<DT, 2>(p, s);
    case 4: return launch_tl<DT, 4>(p, s);
    case 8: return launch_tl<DT, 8>(p, s);
    case 16: return launch_tl<DT, 16>(p, s);
    case 32: return launch_tl<DT, 32>(p, s);
    case 64: return launch_tl<DT, 64>(p, s);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

int launch_compress_keys(const CompressParams &p, void *stream)
{
    return p.dtype == QSA_BF16 ? launch_dt<QSA_BF16>(p, stream) : launch_dt<QSA_F32>(p, stream);
}

}  // namespace qsa
