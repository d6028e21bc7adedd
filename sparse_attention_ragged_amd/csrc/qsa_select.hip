// Block selection: the step after key compression ("QSACompressKeysPaged" names the
// block scorer that re-derives its per-sequence stride; no page gives its contract, so
// the rule below is this library's reading). Row r of sequence b at position pos =
// cache_lengths[b] + (r - row_off[b]) has nfull = (pos + 1) / ratio complete blocks and
// chooses among j < nv = min(nfull, max_blocks). Block j scores q_index[r] .
// block_keys[b * max_blocks + j] (fp32 sum of products); the k = min(topk, nv) highest
// scores are kept, equal scores going to the lower block index. The row's token
// indices are the positions of the kept blocks in increasing order, then its
// incomplete group nfull * ratio .. pos; counts[r] is their number.
//
// Two kernels. Scoring (HBM-bound: each block key read once per row that sees it,
// mostly from L2 when several rows of a sequence share them) gives every block key to
// a team of head_dim * elem / 16 lanes, one 16-byte chunk each, reduced with DPP and
// lane shuffles; a workgroup covers consecutive blocks of one row. Selection runs one
// workgroup per row over the row's scores held in LDS as order-preserving integer
// keys: an MSB-first radix select (up to three digit histograms of 11, 11 and 10 bits
// with LDS atomics, two copies each; it stops once every key left in the chosen bin is
// needed) finds the high bits of the k-th largest key and how many keys sharing them
// are needed; then each thread takes a contiguous segment of candidates, counts its
// keys above that bin and in it, and after one workgroup scan of those counts emits
// its kept blocks at their ranks: every key above the bin and the first needed keys
// in it, already in increasing block order.
#include "qsa_device.hpp"
#include "qsa_select_host.hpp"

namespace qsa {
namespace {

constexpr int kSelThreads = 256;    // scoring kernel
constexpr int kTopkThreads = 1024;  // selection kernel: sixteen wavefronts hide its LDS latency
constexpr int kScoreRounds = 8;      // blocks per team in the scoring kernel (loads in flight)

template <int DT>
__device__ __forceinline__ float dot16(const u32x4 &a, const u32x4 &b)
{
    float s = 0.f;
    if constexpr (DT == QSA_BF16) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            s += bf16_lo(a[w]) * bf16_lo(b[w]) + bf16_hi(a[w]) * bf16_hi(b[w]);
    } else {
#pragma unroll
        for (int w = 0; w < 4; ++w)
            s += __uint_as_float(a[w]) * __uint_as_float(b[w]);
    }
    return s;
}

// Candidate blocks of row r (and the row's sequence and position).
__device__ __forceinline__ int64_t candidates(const SelectParams &p, int64_t r, int &b, int64_t &pos,
                                             int64_t &nfull)
{
    b = find_seq_pos_wave(p.row_off, p.cache_lengths, p.batch, (uint32_t)r, pos);
    nfull = (pos + 1) / p.ratio;
    int64_t nv = nfull < p.max_blocks ? nfull : p.max_blocks;
    return nv < p.cand_bound ? nv : p.cand_bound;
}

template <int DT, int TL>
__global__ __launch_bounds__(kSelThreads) void select_score_kernel(SelectParams p)
{
    constexpr int EB = Elem<DT>::bytes;
    constexpr int TPB = kSelThreads / TL;
    const int64_t per_wg = (int64_t)TPB * kScoreRounds;
    const int64_t wg_per_row = (p.cand_bound + per_wg - 1) / per_wg;
    const int64_t r = blockIdx.x / wg_per_row;
    const int64_t j0 = (int64_t)(blockIdx.x - r * wg_per_row) * per_wg + threadIdx.x / TL;
    const int tl = threadIdx.x % TL;
    int b;
    int64_t pos, nfull;
    const int64_t nv = candidates(p, r, b, pos, nfull);
    if (j0 >= nv)
        return;                                               // whole teams leave together
    const u32x4 q = ldg16(static_cast<const char *>(p.q_index) + (r * p.head_dim) * EB + tl * 16);
    const char *keys = static_cast<const char *>(p.block_keys) + ((int64_t)b * p.max_blocks * p.head_dim) * EB + tl * 16;
    u32x4 k[kScoreRounds];
#pragma unroll
    for (int i = 0; i < kScoreRounds; ++i) {
        const int64_t j = j0 + (int64_t)i * TPB;
        k[i] = ldg16(keys + ((j < nv ? j : j0) * p.head_dim) * EB);
    }
#pragma unroll
    for (int i = 0; i < kScoreRounds; ++i) {
        const int64_t j = j0 + (int64_t)i * TPB;
        const float s = team_sum<TL>(dot16<DT>(q, k[i]));
        if (j < nv && tl == 0)
            p.scores[r * p.cand_bound + j] = s;
    }
}

// binary32 -> unsigned integer with the same order (larger float, larger key).
__device__ __forceinline__ uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over a workgroup of TH threads in thread order (wavefront
// scans with lane shuffles, then the wavefronts' totals through LDS).
template <int TH>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *s_wave)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t u = (uint32_t)__shfl_up((int)inc, off);
        inc += lane >= off ? u : 0u;
    }
    if (lane == 63)
        s_wave[wave] = inc;
    __syncthreads();
    uint32_t before = 0u;
#pragma unroll
    for (int w = 0; w < TH / 64; ++w)
        before += w < wave ? s_wave[w] : 0u;
    return before + inc - v;
}

// The same, also giving the workgroup's total.
template <int TH>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *s_wave, uint32_t &total)
{
    const uint32_t before = block_exclusive_sum<TH>(v, s_wave);
    total = 0u;
#pragma unroll
    for (int w = 0; w < TH / 64; ++w)
        total += s_wave[w];
    return before;
}

template <int CAP>
__global__ __launch_bounds__(kTopkThreads) void select_topk_kernel(SelectParams p)
{
    constexpr int TH = kTopkThreads;
    constexpr int NW = TH / 64;
    constexpr int kBins = 2048;                               // 11-bit digits
    static_assert(2 * TH == kBins, "each thread scans two bins");
    __shared__ uint32_t s_key[CAP];
    // two copies of the digit histogram (even and odd wavefronts) during the radix
    // select; afterwards the kept blocks in rank order (when they fit), so the outputs
    // are written coalesced
    constexpr int kStaged = 2 * kBins;
    __shared__ uint32_t s_hist[2][kBins];
    uint32_t *s_sel = &s_hist[0][0];
    __shared__ uint32_t s_wave[NW];
    __shared__ uint32_t s_digit[3];                           // chosen digit, keys still needed, keys in its bin
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    int b;
    int64_t pos, nfull;
    const int64_t nv = candidates(p, r, b, pos, nfull);
    const int64_t k = p.topk < nv ? p.topk : nv;
    const int64_t tail = pos + 1 - nfull * p.ratio;           // 0 .. ratio - 1
    int32_t *idx = p.token_indices + r * p.width;

    // threshold: the resolved high bits (prefix P under mask M) of the k-th largest key
    // and how many keys with those bits to keep. The passes stop early once every key
    // left in the chosen bin is needed.
    uint32_t P = 0u, M = 0u, need_eq = 0u;
    const bool partial = k > 0 && k < nv;
    if (partial) {
        // eight loads in flight per thread (the loop is otherwise latency-bound)
        constexpr int kInFlight = 8;
        const float *sc = p.scores + r * p.cand_bound;
        for (int64_t i0 = 0; i0 < nv; i0 += kInFlight * TH) {
            float v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int64_t i = i0 + u * TH + tid;
                v[u] = sc[i < nv ? i : 0];
            }
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) {
                const int64_t i = i0 + u * TH + tid;
                if (i < nv)
                    s_key[i] = order_key(v[u]);
            }
        }
        // digits: bits 31..21, 20..10, 9..0
        uint32_t prefix = 0u, mask = 0u, remaining = (uint32_t)k;
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
            const uint32_t dmask = pass == 2 ? 1023u : 2047u;
            for (int i = tid; i < 2 * kBins; i += TH)
                (&s_hist[0][0])[i] = 0u;
            __syncthreads();
            uint32_t *hist = s_hist[wave & 1];
#pragma unroll 8
            for (int64_t i = tid; i < nv; i += TH) {
                const uint32_t key = s_key[i];
                if ((key & mask) == prefix)
                    atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
            __syncthreads();
            // thread t holds bins 2t and 2t + 1; keys in higher bins come from the scan
            const uint32_t h0 = s_hist[0][2 * tid] + s_hist[1][2 * tid];
            const uint32_t h1 = s_hist[0][2 * tid + 1] + s_hist[1][2 * tid + 1];
            uint32_t total;
            const uint32_t below = block_exclusive_sum<TH>(h0 + h1, s_wave, total);
            const uint32_t above1 = total - below - h0 - h1;
            const uint32_t above0 = above1 + h1;
            if (above1 < remaining && above1 + h1 >= remaining) {
                s_digit[0] = (uint32_t)(2 * tid + 1);
                s_digit[1] = remaining - above1;
                s_digit[2] = h1;
            } else if (above0 < remaining && above0 + h0 >= remaining) {
                s_digit[0] = (uint32_t)(2 * tid);
                s_digit[1] = remaining - above0;
                s_digit[2] = h0;
            }
            __syncthreads();
            prefix |= s_digit[0] << shift;
            mask |= dmask << shift;
            remaining = s_digit[1];
            const bool all_of_bin = s_digit[2] == remaining;
            __syncthreads();
            if (all_of_bin)
                break;                            // every key with this prefix is kept
        }
        P = prefix;
        M = mask;
        need_eq = remaining;
    }

    // keep, in block order, every key above T and the first need_eq keys equal to T (all
    // candidates when k == nv). Thread t owns a contiguous segment of candidates: one
    // count pass, one workgroup scan of its (above, equal) counts, one emitting pass.
    if (k > 0) {
        // an odd segment length keeps the threads' LDS reads on distinct banks
        const int64_t seg = ((nv + TH - 1) / TH) | 1;
        const int64_t lo = tid * seg < nv ? tid * seg : nv;
        const int64_t hi = lo + seg < nv ? lo + seg : nv;
        uint32_t gt = 0u, eq = 0u;
        if (partial) {
#pragma unroll 8
            for (int64_t i = lo; i < hi; ++i) {
                const uint32_t key = s_key[i];
                gt += key > (P | ~M) ? 1u : 0u;
                eq += (key & M) == P ? 1u : 0u;
            }
        }
        // both counts fit 16 bits (at most 32768 candidates): scan them packed
        const uint32_t before = block_exclusive_sum<TH>((gt << 16) | eq, s_wave);
        uint32_t eq_seen = before & 0xffffu;
        int64_t m = partial ? (int64_t)(before >> 16) + (eq_seen < need_eq ? eq_seen : need_eq) : lo;
        const bool staged = k <= kStaged;
        for (int64_t i = lo; i < hi; ++i) {
            bool sel = true;
            if (partial) {
                const uint32_t key = s_key[i];
                const bool eq = (key & M) == P;
                sel = key > (P | ~M) || (eq && eq_seen < need_eq);
                eq_seen += eq ? 1u : 0u;
            }
            if (sel) {
                if (staged) {
                    s_sel[m] = (uint32_t)i;
                } else {
                    for (int t = 0; t < p.ratio; ++t)
                        idx[m * p.ratio + t] = (int32_t)(i * p.ratio + t);
                    if (p.blocks)
                        p.blocks[r * p.topk + m] = (int32_t)i;
                }
                ++m;
            }
        }
        if (staged) {
            __syncthreads();
            // k * ratio <= pos + 1: token positions, which the int32 outputs hold
            const uint32_t ratio = (uint32_t)p.ratio;
            for (uint32_t e = tid; e < (uint32_t)(k * p.ratio); e += TH) {
                const uint32_t q = e / ratio;
                idx[e] = (int32_t)(s_sel[q] * ratio + (e - q * ratio));
            }
            if (p.blocks)
                for (int64_t q = tid; q < k; q += TH)
                    p.blocks[r * p.topk + q] = (int32_t)s_sel[q];
        }
    }
    // the incomplete group, the count, and -1 for unused block slots
    for (int64_t t = tid; t < tail; t += TH)
        idx[k * p.ratio + t] = (int32_t)(nfull * p.ratio + t);
    if (tid == 0)
        p.counts[r] = (int32_t)(k * p.ratio + tail);
    if (p.blocks)
        for (int64_t m = k + tid; m < p.topk; m += TH)
            p.blocks[r * p.topk + m] = -1;
}

template <int DT>
int launch_score(const SelectParams &p, hipStream_t s)
{
    const int tl = p.head_dim * Elem<DT>::bytes / 16;
    const int64_t per_wg = (int64_t)(kSelThreads / tl) * kScoreRounds;
    const dim3 grid((unsigned)(p.total_q * ((p.cand_bound + per_wg - 1) / per_wg))), block(kSelThreads);
    switch (tl) {
    case 1: hipLaunchKernelGGL((select_score_kernel<DT, 1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((select_score_kernel<DT, 2>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((select_score_kernel<DT, 4>), grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL((select_score_kernel<DT, 8>), grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL((select_score_kernel<DT, 16>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((select_score_kernel<DT, 32>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((select_score_kernel<DT, 64>), grid, block, 0, s, p); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // namespace

int launch_select_blocks(const SelectParams &p, void *stream, void *ev_start, void *ev_stop)
{
    if (p.total_q == 0)
        return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int err = 0;
    if (ev_start)
        err = (int)hipEventRecord(static_cast<hipEvent_t>(ev_start), s);
    if (!err && p.cand_bound > 0)
        err = p.dtype == QSA_BF16 ? launch_score<QSA_BF16>(p, s) : launch_score<QSA_F32>(p, s);
    if (!err) {
        const dim3 grid((unsigned)p.total_q), block(kTopkThreads);
        if (p.cand_bound <= 4096)
            hipLaunchKernelGGL(select_topk_kernel<4096>, grid, block, 0, s, p);
        else
            hipLaunchKernelGGL(select_topk_kernel<kSelectMaxCandidates>, grid, block, 0, s, p);
        err = (int)hipGetLastError();
    }
    if (!err && ev_stop)
        err = (int)hipEventRecord(static_cast<hipEvent_t>(ev_stop), s);
    return err;
}

}  // namespace qsa
