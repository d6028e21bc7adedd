// Dense ragged attention on matrix cores with key tiles shared by several query rows
// ("RaggedFlashAttentionGPU": summary, Parameters and Args; bf16, groups of 8 or 16
// query heads per kv head, no split).
//
// A workgroup of 4 wavefronts takes 8 consecutive rows of the ragged batch (4 at
// head_dim 256) and one kv head; wavefront w owns rows r0 + 2w and r0 + 2w + 1 (their
// 16 query heads fill the M side of the 16x16x32 MFMAs, as in the gather kernel, and
// each K or V fragment read from LDS feeds the MFMAs of both rows). Row i of sequence b sees the keys lo..hi of
// its own sequence, which sit at consecutive rows of the ragged k and v; the union of
// the workgroup's rows' ranges is one contiguous range of global rows (sequences are
// contiguous in the ragged layout), so the workgroup walks that range in tiles of 32
// keys. Each tile's K and V rows are loaded once by all four wavefronts together (8
// rows each, 16 bytes a lane, row-contiguous) into one of two LDS buffers; every
// wavefront then computes its own rows' scores over the tile (keys outside a row's
// range masked), the online softmax in the log2 domain and P.V, exactly as the gather
// kernel does for a tile of its own. One barrier per tile: the rows of the next two
// tiles are in flight while the current one is consumed, and the next one is written
// to the other buffer.
//
// Compared with one wavefront per row walking its keys alone, the L2-to-LDS traffic and
// the address work drop by the number of rows sharing a tile (8), and the LDS reads by
// the rows per wavefront (2); the MFMA work is the same.
#include <type_traits>

#include "qsa_device.hpp"
#include "qsa_flash_host.hpp"

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int kFlashWaves = 4;       // rows (and wavefronts) per workgroup
constexpr int kFlashTile = 32;       // keys per tile
constexpr float kFlashSlack = 8.0f;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v)
{
    bf16x8_t r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

// Rows per wavefront: two at head_dim <= 128 (each K and V fragment read from LDS then
// feeds both rows' MFMAs), one above (register budget).
template <int D>
constexpr int flash_rows_per_wave() { return D <= 128 ? 2 : 1; }

template <int D>
__global__ void __launch_bounds__(64 * kFlashWaves) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
gather_mfma_flash_kernel(GatherParams p)
{
    constexpr int EB = 2;                       // bf16
    constexpr int NC = D / 32;                  // 32-dim chunks of QK^T
    constexpr int NDT = D / 16;                 // 16-dim tiles of the output
    constexpr int RW = flash_rows_per_wave<D>();
    constexpr int ROWS = kFlashWaves * RW;      // rows per workgroup
    constexpr int RB = D * EB;                  // bytes of one K (or V) row
    constexpr int LPK = RB / 16;                // lanes that load one row
    constexpr int KPI = 64 / LPK;               // rows per load instruction
    constexpr int RPW = kFlashTile / kFlashWaves;   // rows of a tile each wavefront loads
    constexpr int NI = RPW / KPI;               // load instructions per plane, tile and wavefront
    constexpr int KROWB = RB + 32;              // LDS row of the K tile (bytes), padded
    constexpr int VROW = D + 16;                // LDS row of the V tile (bf16 elements), padded
    constexpr int kBufBytes = kFlashTile * (KROWB + 2 * VROW);
    static_assert(D % 32 == 0 && LPK >= 1 && LPK <= 64 && RPW % KPI == 0 && NI >= 1, "unsupported head_dim");
    __shared__ __attribute__((aligned(16))) char smem[2 * kBufBytes];
    __shared__ int64_t s_range[ROWS][2];

    const int G = p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lq = lane >> 4;

    // workgroup -> (row block, kv head), kv heads fastest and row blocks from the last:
    // blocks are dealt to the XCDs round-robin, so every XCD gets an even share of early
    // and late (causal: short and long) rows, and the longest blocks start first
    const int64_t nblk = (p.total_q + ROWS - 1) / ROWS;
    const int g = (int)(blockIdx.x % (uint32_t)p.num_kv_heads);
    const int64_t r0 = (nblk - 1 - (int64_t)(blockIdx.x / (uint32_t)p.num_kv_heads)) * ROWS;

    // this wavefront's rows r0 + RW*wave + j: q fragments, key ranges [first, first + n)
    const bool head_real = li < G;
    u32x4 qf[RW][NC];
    int64_t first[RW], n[RW];
    bool row_real[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int64_t r = r0 + RW * wave + j;
        row_real[j] = r < p.total_q;
        const int64_t rr = row_real[j] ? r : r0;  // a real row to read for padding
        const char *qrow0 = static_cast<const char *>(p.q) + ((rr * p.num_q_heads + (int64_t)g * G) * D) * EB;
        const char *qrow = head_real ? qrow0 + (int64_t)li * D * EB : qrow0;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4 v = ldg16(qrow + (32 * c + 8 * lq) * EB);
            qf[j][c] = head_real ? v : u32x4{0, 0, 0, 0};
        }
        first[j] = 0;
        const int b = find_seq_pos_wave(p.row_off, nullptr, p.batch, (uint32_t)rr, first[j]);
        n[j] = row_real[j] ? dense_key_range(p, rr, b, first[j]) : 0;
        if (lane == 0) {
            s_range[RW * wave + j][0] = n[j] > 0 ? first[j] : INT64_MAX;
            s_range[RW * wave + j][1] = n[j] > 0 ? first[j] + n[j] : INT64_MIN;
        }
    }
    __syncthreads();
    int64_t K0 = INT64_MAX, K1 = INT64_MIN;
#pragma unroll
    for (int w = 0; w < ROWS; ++w) {
        K0 = s_range[w][0] < K0 ? s_range[w][0] : K0;
        K1 = s_range[w][1] > K1 ? s_range[w][1] : K1;
    }
    // Row indices, key ranges and tile starts in 32 bits (total_q < 2^31 is checked on
    // the host; a prefetched tile past the range stays below 2^32), each the same in
    // every lane and taken from lane 0, so that the per-tile range tests are scalar.
    const uint32_t K0u = K1 > K0 ? (uint32_t)__builtin_amdgcn_readfirstlane((int)K0) : 0u;
    const uint32_t K1u = K1 > K0 ? (uint32_t)__builtin_amdgcn_readfirstlane((int)K1) : 0u;
    const int nt = (int)((K1u - K0u + kFlashTile - 1) / kFlashTile);
    uint32_t fu[RW], nu[RW];                     // each row's first key and key count
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        fu[j] = (uint32_t)__builtin_amdgcn_readfirstlane((int)first[j]);
        nu[j] = (uint32_t)__builtin_amdgcn_readfirstlane((int)n[j]);
    }

    // softmax state per row: reference m (log2 units) of head li, the P.V accumulator
    // and the running sum of the weights, kept by an MFMA with an all-ones A operand
    // (every element of lsum[j] is the sum over the row's keys for head li, of the same
    // bf16-rounded weights that P.V uses)
    float m[RW];
    f32x4_t acc[RW][NDT], lsum[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        m[j] = kNoKey;
        lsum[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NDT; ++t)
            acc[j][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs
    // with a positive scale the maximum of the scaled scores is the scaled maximum, so
    // the scale is applied once to the maximum and folded into the exponent's FMA (the
    // tile loop is compiled for both cases and chosen once per call)

    // loading layout: wavefront w loads rows RPW*w .. RPW*w + RPW-1 of each tile
    const int my_row = lane / LPK;
    const int my_chunk = lane % LPK;
    const char *kbase = static_cast<const char *>(p.dense_k) + ((int64_t)g * D) * EB + my_chunk * 16;
    const char *vbase = static_cast<const char *>(p.dense_v) + ((int64_t)g * D) * EB + my_chunk * 16;
    const uint32_t row_stride = (uint32_t)p.num_kv_heads * D * EB;
    struct Rows { u32x4 k[NI], v[NI]; };
    auto load_tile = [&](int t, Rows &R) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t kg = K0u + (uint32_t)t * kFlashTile + (uint32_t)(RPW * wave + i * KPI + my_row);
            const uint32_t kr = kg < K1u ? kg : K1u - 1;   // past the range: its last row (readable)
            const uint64_t off = (uint64_t)kr * row_stride;
            R.k[i] = ldg16(kbase + off);
            R.v[i] = ldg16(vbase + off);
        }
    };
    auto store_tile = [&](int buf, const Rows &R) {
        char *s_k = smem + buf * kBufBytes;
        uint16_t *s_v = reinterpret_cast<uint16_t *>(s_k + kFlashTile * KROWB);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = RPW * wave + i * KPI + my_row;
            *reinterpret_cast<u32x4 *>(s_k + row * KROWB + my_chunk * 16) = R.k[i];
            *reinterpret_cast<u32x4 *>(s_v + row * VROW + my_chunk * 8) = R.v[i];
        }
    };
    auto consume = [&](int t, int buf, auto fold_c) {
        constexpr bool fold = decltype(fold_c)::value;
        const uint32_t t0 = K0u + (uint32_t)t * kFlashTile;
        bool any = false;
#pragma unroll
        for (int j = 0; j < RW; ++j)
            any = any || (t0 < fu[j] + nu[j] && t0 + kFlashTile > fu[j]);
        if (!any)
            return;                               // no key of these rows in the tile
        const char *s_k = smem + buf * kBufBytes;
        const uint16_t *s_v = reinterpret_cast<const uint16_t *>(s_k + kFlashTile * KROWB);
        // S^T (two 16-key halves) for every row: each K fragment feeds all rows' MFMAs
        f32x4_t st[RW][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int j = 0; j < RW; ++j)
                st[j][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const char *kp = s_k + (16 * h + li) * KROWB + (32 * c + 8 * lq) * EB;
                const bf16x8_t ka = as_bf16x8(*reinterpret_cast<const u32x4 *>(kp));
#pragma unroll
                for (int j = 0; j < RW; ++j)
                    st[j][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, as_bf16x8(qf[j][c]), st[j][h], 0, 0, 0);
            }
        }
        // per row: scores in the log2 domain (keys outside the row's range at -inf),
        // online softmax, P^T as the B operand
        u32x4 pb[RW];
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            // key index relative to the row's first key; a tile wholly inside the
            // row's range (all but its first and last few) needs no mask
            const int32_t rel0 = (int32_t)(t0 - fu[j]);
            const bool whole = rel0 >= 0 && rel0 + kFlashTile <= (int32_t)nu[j];
            float sc[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sc[h][i] = fold ? st[j][h][i] : st[j][h][i] * p.scale_log2;
            if (!whole) {
                const int32_t rel = rel0 < -kFlashTile ? -kFlashTile : rel0 > (int32_t)nu[j] ? (int32_t)nu[j] : rel0;
                const uint32_t nn = nu[j];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sc[h][i] = (uint32_t)(rel + 16 * h + 4 * lq + i) < nn ? sc[h][i] : kNegInf;
            }
            float mx = score_max(score_max(score_max(sc[0][0], sc[0][1]), score_max(sc[0][2], sc[0][3])),
                                 score_max(score_max(sc[1][0], sc[1][1]), score_max(sc[1][2], sc[1][3])));
            mx = xor32_max(xor16_max(mx));
            mx = score_max(fold ? mx * p.scale_log2 : mx, m[j]);
            if (__any(mx > m[j] + kFlashSlack)) {
                const float alpha = __builtin_amdgcn_exp2f(m[j] - mx);
                lsum[j] *= alpha;
#pragma unroll
                for (int u = 0; u < NDT; ++u)
                    acc[j][u] *= alpha;
                m[j] = mx;
            }
            float w[2][4];
            const float sl = fold ? p.scale_log2 : 1.f;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[h][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[h][i], sl, -m[j]));
            // k-slot t < 4 is key 4q + t, t >= 4 is key 16 + 4q + t - 4
            pb[j] = u32x4{pack_bf16x2(w[0][0], w[0][1]), pack_bf16x2(w[0][2], w[0][3]),
                          pack_bf16x2(w[1][0], w[1][1]), pack_bf16x2(w[1][2], w[1][3])};
            lsum[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), as_bf16x8(pb[j]), lsum[j], 0, 0, 0);
        }
        // V^T as the A operand via transposing LDS reads, shared by every row
        const int jr = li >> 2, qd = li & 3;
#pragma unroll
        for (int u = 0; u < NDT; ++u) {
            const int col = 16 * u + 4 * qd;
            const s16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(s_v + (4 * lq + jr) * VROW + col));
            const s16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(s_v + (16 + 4 * lq + jr) * VROW + col));
            u32x4 av;
            __builtin_memcpy(&av, &a0, 8);
            __builtin_memcpy(reinterpret_cast<char *>(&av) + 8, &a1, 8);
#pragma unroll
            for (int j = 0; j < RW; ++j)
                acc[j][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(pb[j]), acc[j][u], 0, 0, 0);
        }
    };

    // two tiles in flight: tile t + 2 is loaded while tile t is consumed and tile t + 1
    // (loaded one iteration earlier) goes to the other LDS buffer; one barrier per tile.
    // Loads and stores are unconditional (a tile past the range reads the range's first
    // rows and is never consumed), and every trip starts with the same two register sets
    // in flight, so the compiler's wait counts keep the newer tile's loads in flight
    // instead of draining them.
    auto tiles = [&](auto fold_c) {
        Rows R0, R1;
        load_tile(0, R0);
        load_tile(1, R1);
        for (int t = 0;; t += 2) {
            store_tile(0, R0);                    // tile t
            lds_barrier();
            load_tile(t + 2, R0);
            consume(t, 0, fold_c);
            store_tile(1, R1);                    // tile t + 1
            lds_barrier();
            if (t + 1 >= nt)
                break;
            load_tile(t + 3, R1);
            consume(t + 1, 1, fold_c);
            if (t + 2 >= nt)
                break;
        }
    };
    if (nt > 0) {
        if (p.scale_log2 > 0.f)
            tiles(std::true_type());
        else
            tiles(std::false_type());
    }

    // Per-head sums over the four lanes of each head. Lane (i, q) holds dims 16u + 4q ..
    // 16u + 4q + 3 of head i, so a direct store would write 32- or 64-byte pieces of up to
    // 16 rows per instruction; each row's values pass through this wavefront's own part
    // of LDS tile buffer 0 (16 head slots x D bytes, padded by 16), which nobody reads
    // after the tile loop's last barrier, so that every store writes whole 16-byte chunks
    // of one output row, D bytes of a head per pass (two passes of bf16, four of fp32).
    {
        constexpr int RS = D + 16;              // staging bytes per head slot
        constexpr int CPR = D / 16;             // 16-byte chunks per head and pass
        static_assert(kFlashWaves * 16 * RS <= kBufBytes, "the staging rows fit tile buffer 0");
        static_assert(D % 64 == 0, "whole wavefront stores");
        char *stage = smem + wave * 16 * RS;
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const float ls = lsum[j][0];
            const int64_t head0 = (int64_t)g * G;
            const float f = li < G ? final_factor(p, head0 + li, m[j], ls) : 0.f;
            const int64_t row = r0 + RW * wave + j;
            auto emit = [&](auto ob) {
                constexpr int OB = decltype(ob)::value;
                constexpr int PT = D / OB / 16;     // MFMA tiles per pass
                char *dst0 = static_cast<char *>(p.out) + (row * p.num_q_heads + head0) * (int64_t)D * OB;
#pragma unroll
                for (int pass = 0; pass < OB; ++pass) {
                    asm volatile("" ::: "memory");  // after the previous reads of this region
#pragma unroll
                    for (int tl = 0; tl < PT; ++tl) {
                        const f32x4_t v = acc[j][pass * PT + tl] * f;
                        char *a = stage + li * RS + (16 * tl + 4 * lq) * OB;
                        if constexpr (OB == 2) {
                            typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
                            *reinterpret_cast<u32x2v *>(a) = u32x2v{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        } else {
                            *reinterpret_cast<f32x4_t *>(a) = v;
                        }
                    }
                    asm volatile("" ::: "memory");  // the reads below take other lanes' values
#pragma unroll
                    for (int q4 = 0; q4 < D / 64; ++q4) {
                        const int c = q4 * 64 + lane;
                        const int hh = c / CPR, q = c % CPR;
                        const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + hh * RS + q * 16);
                        if (row_real[j] && hh < G)
                            *reinterpret_cast<u32x4 *>(dst0 + (int64_t)hh * D * OB + pass * D + q * 16) = v;
                    }
                }
            };
            if (p.out_dtype == QSA_BF16)
                emit(std::integral_constant<int, 2>{});
            else
                emit(std::integral_constant<int, 4>{});
        }
    }
}

template <int D>
int launch_flash(const GatherParams &p, void *stream)
{
    constexpr int ROWS = kFlashWaves * flash_rows_per_wave<D>();
    const int64_t nblk = (p.total_q + ROWS - 1) / ROWS;
    const int64_t grid = nblk * p.num_kv_heads;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gather_mfma_flash_kernel<D>), dim3((unsigned)grid), dim3(64 * kFlashWaves), 0,
                       static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace

int launch_gather_mfma_flash(const GatherParams &p, void *stream)
{
    switch (p.head_dim) {
    case 64: return launch_flash<64>(p, stream);
    case 128: return launch_flash<128>(p, stream);
    case 256: return launch_flash<256>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace qsa
