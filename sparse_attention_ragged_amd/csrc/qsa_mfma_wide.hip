// Latent gather-attention on matrix cores for wide head groups ("latent_sparse_attention_
// ragged_paged": one latent head whose row is both key and value, many query heads).
//
// One workgroup owns one (query row, split) and has one wavefront per tile of 16 query
// heads (up to 64 heads, head_dim up to 512). The keys of the split (window positions,
// then listed compressed entries) go through the three-stage address pipeline and
// arrive 32 at a time in an LDS tile that all wavefronts share; the next tile's rows
// are in flight while the current one is used (two LDS buffers, one barrier per tile).
// Each wavefront then runs, on 16x16x32 MFMAs,
//   S^T = X . Q^T    (A: 8 dims of key i from LDS, B: its heads' q rows, held in VGPRs)
//   online softmax per head in the log2 domain (lazy rescale as in the other kernels)
//   O^T += X^T P^T   (A: transposing LDS reads of the same tile, B: P^T straight from
//                     the S^T accumulators)
// and owns its heads' whole output rows, so no cross-wave merge is needed. The per-head
// sink logit joins the denominator once, at the final normalisation (here with one
// split, in the combine kernel otherwise).
#include "qsa_device.hpp"

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int kWideMaxWaves = 4;      // 64 heads
constexpr int kWTile = 32;            // keys per tile
constexpr float kWSlack = 8.0f;
constexpr int kWThreads = 64 * kWideMaxWaves;

__device__ __forceinline__ bf16x8_t wide_bf16x8(u32x4 v)
{
    bf16x8_t r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

template <int D, int WAVES>
__global__ void __launch_bounds__(kWThreads) gather_mfma_wide_kernel(GatherParams p)
{
    constexpr int EB = 2;                       // bf16
    constexpr int NC = D / 32;
    constexpr int NDT = D / 16;
    constexpr int ROW = D + 8;                  // LDS row (bf16 elements), +16 B against bank conflicts
    constexpr int CHUNKS = D * EB / 16;         // 16-byte chunks of one row
    static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
    __shared__ __attribute__((aligned(16))) uint16_t s_x[2][kWTile * ROW];
    __shared__ uint32_t s_ok[2];

    const int S = p.num_splits;
    const int G = p.group;
    const int s = (int)(blockIdx.x % S);
    const int64_t r = blockIdx.x / S;
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lq = lane >> 4;

    // staging layout: tpk threads per key, each loading cpt chunks (chunk u*tpk + sub)
    constexpr int tpk = 64 * WAVES / kWTile;
    constexpr int cpt = CHUNKS / tpk;
    static_assert(CHUNKS % tpk == 0, "row chunks must split evenly over a key's threads");
    const int skey = tid / tpk;
    const int ssub = tid % tpk;
    (void)nthreads;

    // prologue
    const int64_t n = key_list_length(p, r);
    const int head = 16 * wave + li;            // within the group
    const bool head_real = head < G;
    const char *qrow0 = static_cast<const char *>(p.q) + (r * p.num_q_heads) * D * EB;
    const char *qrow = head_real ? qrow0 + (int64_t)head * D * EB : qrow0;
    u32x4 qf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const u32x4 v = ldg16(qrow + (32 * c + 8 * lq) * EB);
        qf[c] = head_real ? v : u32x4{0, 0, 0, 0};
    }
    const int b = find_seq_wave(p.row_off, p.batch, (uint32_t)r);
    const int64_t pos = (int64_t)p.cache_lengths[b] + (r - (int64_t)p.row_off[b]);
    const int64_t j0 = (int64_t)s * p.split_keys;
    const int64_t j1 = n < j0 + p.split_keys ? n : j0 + p.split_keys;
    const int nb = j1 > j0 ? (int)((j1 - j0 + kWTile - 1) / kWTile) : 0;
    const char *dummy = qrow0;

    float m = kNoKey, lsum = 0.f;
    f32x4_t acc[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t)
        acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    struct Entry { int32_t raw; };
    struct Page { KeyPos k; int32_t slot; uint32_t page; };
    struct Rows { u32x4 x[cpt]; bool ok; };

    auto key_index = [&](int tile) -> int64_t { return j0 + (int64_t)tile * kWTile + skey; };
    auto load_entry = [&](int tile, Entry &E) {
        const int64_t jj = key_index(tile);
        E.raw = *entry_ptr<KEYS_LATENT>(p, r, 0, jj, jj < j1);
    };
    auto load_page = [&](int tile, const Entry &E, Page &P) {
        const int64_t jj = key_index(tile);
        P.k = key_pos<KEYS_LATENT>(p, pos, jj, E.raw, jj < j1);
        P.page = *page_entry_ptr(p, b, P.k, P.slot);
    };
    auto load_rows = [&](const Page &P, Rows &R) {
        bool ok;
        const char *a = row_address<EB, KEYS_LATENT>(p, P.k, P.page, P.slot, 0, dummy, ok);
        R.ok = ok;
        const char *base = ok ? a : dummy;
#pragma unroll
        for (int u = 0; u < cpt; ++u)
            R.x[u] = ldg16(base + (int64_t)(u * tpk + ssub) * 16);
    };
    auto store_rows = [&](const Rows &R, int buf) {
        uint16_t *row = s_x[buf] + skey * ROW;
#pragma unroll
        for (int u = 0; u < cpt; ++u)
            *reinterpret_cast<u32x4 *>(row + (u * tpk + ssub) * 8) = R.x[u];
        if (ssub == 0) {
            const unsigned long long bal = __ballot(R.ok);
            // keys of this wavefront: lanes 0, tpk, 2 tpk, ... hold them in order
            uint32_t bits = 0;
            for (int k = 0; k < 64 / tpk; ++k)
                bits |= (uint32_t)((bal >> (k * tpk)) & 1ull) << k;
            if (lane == 0)
                atomicOr(&s_ok[buf], bits << (wave * (64 / tpk)));
        }
    };
    auto compute = [&](int buf) {
        const uint16_t *x = s_x[buf];
        const uint32_t present = s_ok[buf];
        f32x4_t st[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            st[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 kf = *reinterpret_cast<const u32x4 *>(x + (16 * h + li) * ROW + 32 * c + 8 * lq);
                st[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wide_bf16x8(kf), wide_bf16x8(qf[c]), st[h], 0,
                                                                0, 0);
            }
        }
        float sc[2][4];
        float mx = m;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = 16 * h + 4 * lq + i;
                const float v = st[h][i] * p.scale_log2;
                sc[h][i] = (present >> key) & 1u ? v : kNegInf;
                mx = fmaxf(mx, sc[h][i]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any(mx > m + kWSlack)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mx);
            lsum *= alpha;
#pragma unroll
            for (int t = 0; t < NDT; ++t)
                acc[t] *= alpha;
            m = mx;
        }
        float w[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[h][i] = __builtin_amdgcn_exp2f(sc[h][i] - m);
                lsum += w[h][i];
            }
        const u32x4 pb = {pack_bf16x2(w[0][0], w[0][1]), pack_bf16x2(w[0][2], w[0][3]),
                          pack_bf16x2(w[1][0], w[1][1]), pack_bf16x2(w[1][2], w[1][3])};
        const int jr = li >> 2, qd = li & 3;
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
            const int col = 16 * t + 4 * qd;
            const s16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(x + (4 * lq + jr) * ROW + col));
            const s16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(x + (16 + 4 * lq + jr) * ROW + col));
            u32x4 av;
            __builtin_memcpy(&av, &a0, 8);
            __builtin_memcpy(reinterpret_cast<char *>(&av) + 8, &a1, 8);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wide_bf16x8(av), wide_bf16x8(pb), acc[t], 0, 0, 0);
        }
    };

    if (nb > 0) {
        Entry E0, E1;
        Page P0, P1;
        Rows R;
        if (tid < 2)
            s_ok[tid] = 0;
        __syncthreads();
        load_entry(0, E0);
        load_entry(1, E1);
        load_page(0, E0, P0);
        load_rows(P0, R);
        load_entry(2, E0);
        load_page(1, E1, P1);
        store_rows(R, 0);
        __syncthreads();
        // iteration i: rows(i+1) in flight while tile i is used; entries / pages run
        // two / one tiles ahead of the rows
        for (int i = 0; i < nb; i += 2) {
            load_rows(P1, R);                   // tile i+1
            load_entry(i + 3, E1);
            load_page(i + 2, E0, P0);
            compute(0);
            __syncthreads();                    // every wavefront is done with buffer 0
            if (tid == 0)
                s_ok[0] = 0;
            store_rows(R, 1);
            __syncthreads();
            if (i + 1 >= nb)
                break;
            load_rows(P0, R);                   // tile i+2
            load_entry(i + 4, E0);
            load_page(i + 3, E1, P1);
            compute(1);
            __syncthreads();
            if (tid == 0)
                s_ok[1] = 0;
            store_rows(R, 0);
            __syncthreads();
        }
    }

    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    const int64_t gh = (int64_t)head;           // the single kv head: group = all q heads
    if (head_real) {
        const int64_t rh = r * p.num_q_heads + gh;
        if (S == 1) {
            const float inv = final_factor(p, gh, m, lsum);
#pragma unroll
            for (int t = 0; t < NDT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    store_out(p.out, p.out_dtype, rh * D + 16 * t + 4 * lq + i, acc[t][i] * inv);
        } else {
            const int64_t srh = (int64_t)s * p.total_q * p.num_q_heads + rh;
#pragma unroll
            for (int t = 0; t < NDT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.ws_acc[srh * D + 16 * t + 4 * lq + i] = acc[t][i];
            if (lq == 0) {
                p.ws_ml[srh * 2] = m;
                p.ws_ml[srh * 2 + 1] = lsum;
            }
        }
    }
}

template <int D>
int launch_wide(const GatherParams &p, void *stream)
{
    // one wavefront per 16 heads, rounded up to 2 or 4 wavefronts (padded heads idle)
    const int64_t grid = p.total_q * (int64_t)p.num_splits;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    if (p.group <= 32)
        hipLaunchKernelGGL((gather_mfma_wide_kernel<D, 2>), dim3((unsigned)grid), dim3(128), 0,
                           static_cast<hipStream_t>(stream), p);
    else
        hipLaunchKernelGGL((gather_mfma_wide_kernel<D, 4>), dim3((unsigned)grid), dim3(256), 0,
                           static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace

bool mfma_wide_supported(int32_t dtype, int32_t group, int32_t head_dim, int32_t list_kind)
{
    return dtype == QSA_BF16 && list_kind == KEYS_LATENT && group > 16 && group <= 16 * kWideMaxWaves &&
           (head_dim == 128 || head_dim == 256 || head_dim == 512);
}

int launch_gather_mfma_wide(const GatherParams &p, void *stream)
{
    switch (p.head_dim) {
    case 128: return launch_wide<128>(p, stream);
    case 256: return launch_wide<256>(p, stream);
    case 512: return launch_wide<512>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace qsa
