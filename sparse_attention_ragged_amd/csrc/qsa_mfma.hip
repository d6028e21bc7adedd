// Gather-attention on matrix cores (groups of 8 or 16 query heads per kv head).
//
// Each wavefront owns one (query row, kv head, split) item and walks its keys in tiles
// of 32, so no wavefront ever waits for or merges with another; it normalises and
// stores its own output rows. Items are ordered kv head, row, split (split fastest), a
// workgroup takes NW consecutive items, and workgroups are renumbered so that each of
// the 8 XCDs walks a contiguous range of them: at any time an XCD works on neighbouring
// rows of one kv head, whose selected keys largely coincide and stay in its L2.
// Per tile, with gfx950 16x16x32 MFMAs (lane l: i = l % 16, q = l / 16):
//
//  * loads          lane l walks key l % 32 of the tile through the address pipeline;
//                    the K and V rows are then loaded row-contiguous (one load
//                    instruction covers whole rows, 16 bytes a lane, each lane taking
//                    its row's address from the lane that computed it) and written to
//                    the wavefront's own LDS tiles. (Loading straight into the MFMA
//                    fragment layout touches 16 rows x 64 bytes per instruction and
//                    measured at well under half the L2 gather rate.)
//  * S^T = K . Q^T   A = 16 keys x 32 dims of K from the LDS tile (lane holds 8
//                    consecutive dims of key i), B = Q^T (8 dims of head i, loaded
//                    once). Two key halves x head_dim/32 chunks of MFMAs; C holds, per
//                    lane, keys 4q..4q+3 (+16) of head i.
//  * softmax         per head i, over the four lanes sharing i, in the log2 domain
//                    with the same lazy rescale as the wavefront kernel.
//  * O^T += V^T P^T  B = P^T comes straight out of the S^T accumulator layout (the
//                    MFMA's key order is chosen to match it); A = V^T is read from an
//                    LDS copy of the V tile with the transposing 64-bit LDS load, one
//                    read per 4 keys x 16 dims.
//
// fp8 e4m3 ("Struct_msa_attention_ragged_paged": scale-free FP8, FP32 accumulation):
// S^T uses the fp8 MFMA on the raw codes; V is widened to bf16 (exactly) on its way
// into LDS, so P stays bf16 in P.V. Groups below 16 pad the head dimension of the
// MFMA with zero query rows whose results are dropped.
//
// Keys reach their rows through the same three-stage address pipeline as the
// wavefront kernel (list entry -> page-table entry -> rows), issued a tile ahead.
// Softmax reductions over the four lanes of a head use the gfx950 row-swap permutes.
#include <type_traits>

#include "qsa_device.hpp"

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) u32x2 global_u32x2;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

constexpr int kMfmaMaxWaves = 4;
constexpr int kNumXcd = 8;            // XCDs of an MI355X; blocks are dealt to them round-robin
constexpr int kTileKeys = 32;
constexpr float kSlack = 8.0f;

__device__ __forceinline__ u32x2 ldg8(const void *p) { return *(global_u32x2 *)(p); }

__device__ __forceinline__ long as_long(u32x2 v)
{
    long r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v)
{
    bf16x8_t r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

// 8 e4m3 codes -> 8 bf16 (exact: every e4m3 value is a bf16 value), two codes per
// gfx950 scaled conversion with a scale of 1
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w)
{
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH);
    uint32_t u;
    __builtin_memcpy(&u, &v, sizeof u);
    return u;
}
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 w)
{
    return u32x4{e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]), e4m3x2_to_bf16x2<false>(w[1]),
                 e4m3x2_to_bf16x2<true>(w[1])};
}

template <int DT, int D, int LIST>
__global__ void __launch_bounds__(64 * kMfmaMaxWaves) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
gather_mfma_kernel(GatherParams p)
{
    constexpr int EB = Elem<DT>::bytes;
    constexpr int NC = D / 32;                  // 32-dim chunks of QK^T
    constexpr int NDT = D / 16;                 // 16-dim tiles of the output
    constexpr int RB = D * EB;                  // bytes of one K (or V) row in the cache
    constexpr int LPK = RB / 16;                // lanes that load one row (16 bytes each)
    constexpr int KPI = 64 / LPK;               // rows per load instruction
    constexpr int NI = kTileKeys / KPI;         // load instructions per plane and tile
    // LDS row of the K tile (bytes), padded so that the 16 rows one MFMA fragment read
    // touches fall on distinct banks: bf16 reads 16 bytes a lane (row stride 72 dwords
    // at D 128), e4m3 8 bytes (stride 36 dwords: 16 distinct multiples of 4 mod 64)
    constexpr int KROWB = RB + (EB == 1 ? 16 : 32);
    constexpr int VROW = D + 16;                // LDS row of the V tile (bf16 elements), padded
    constexpr int kWaveLds = kTileKeys * (KROWB + 2 * VROW + 16);   // + (K row, V row) address per key
    static_assert(D % 32 == 0 && LPK >= 1 && LPK <= 64 && kTileKeys % KPI == 0, "unsupported head_dim");
    using Chunk = typename std::conditional<DT == QSA_BF16, u32x4, u32x2>::type;
    __shared__ __attribute__((aligned(16))) char smem[kMfmaMaxWaves * kWaveLds];

    const int S = p.num_splits;
    const int G = p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: the item's indices follow
    const int NW = blockDim.x >> 6;

    // XCD-contiguous renumbering of the workgroups (blocks are dealt to the 8 XCDs
    // round-robin): XCD x takes a contiguous share of the item range
    const int64_t nwg = gridDim.x;
    const int64_t xq = nwg / kNumXcd, xr = nwg % kNumXcd;
    const int64_t xcd = blockIdx.x % kNumXcd, xk = blockIdx.x / kNumXcd;
    const int64_t wg = xcd * xq + (xcd < xr ? xcd : xr) + xk;
    // this wavefront's item: (kv head, row, split), split fastest
    const int64_t item = wg * NW + wave;
    if (item >= p.total_q * (int64_t)p.num_kv_heads * S)
        return;
    const int s = (int)(item % S);
    const int64_t r = (item / S) % p.total_q;
    const int g = (int)(item / S / p.total_q);

    const int li = lane & 15;
    const int lq = lane >> 4;
    char *s_k = smem + wave * kWaveLds;                                     // [32][KROWB] bytes
    uint16_t *s_v = reinterpret_cast<uint16_t *>(s_k + kTileKeys * KROWB);   // [32][VROW] bf16
    u64x2 *s_rows = reinterpret_cast<u64x2 *>(s_k + kTileKeys * (KROWB + 2 * VROW));   // [32] row addresses

    // prologue: list length, sequence and the q fragments go out together
    int64_t n = LIST == KEYS_DENSE ? 0 : key_list_length(p, r);
    const char *qrow0 = static_cast<const char *>(p.q) + ((r * p.num_q_heads + (int64_t)g * G) * D) * EB;
    const bool head_real = li < G;
    const char *qrow = head_real ? qrow0 + (int64_t)li * D * EB : qrow0;
    Chunk qf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if constexpr (DT == QSA_BF16) {
            const u32x4 v = ldg16(qrow + (32 * c + 8 * lq) * EB);
            qf[c] = head_real ? v : u32x4{0, 0, 0, 0};
        } else {
            const u32x2 v = ldg8(qrow + (32 * c + 8 * lq) * EB);
            qf[c] = head_real ? v : u32x2{0, 0};
        }
    }
    const int64_t j0 = (int64_t)s * p.split_keys;
    const int64_t jend = j0 + p.split_keys;
    int64_t j1 = n < jend ? n : jend;            // dense: set once the row's sequence is known

    // Lane l (and l + 32) walks key l % 32 of each tile through the address pipeline.
    // The list entries do not depend on the row's sequence, so the first two tiles'
    // entries are loaded before its lookup.
    const int kl = lane & 31;
    struct Entries { int32_t raw; };
    auto key_index = [&](int batch) -> int64_t { return j0 + (int64_t)batch * kTileKeys + kl; };
    auto load_entries = [&](int batch, Entries &E) {
        const int64_t jj = key_index(batch);
        if constexpr (LIST == KEYS_DENSE)
            E.raw = 0;                             // dense: the key is its index, nothing to load
        else
            E.raw = *entry_ptr<LIST>(p, r, g, jj, jj < j1);
    };
    Entries E0, E1;
    load_entries(0, E0);
    load_entries(1, E1);

    int64_t pos = 0;
    const int b = find_seq_pos_wave(p.row_off,
                                    LIST == KEYS_TOKEN_INDICES || LIST == KEYS_DENSE ? nullptr : p.cache_lengths,
                                    p.batch, (uint32_t)r, pos);
    if constexpr (LIST == KEYS_DENSE) {
        n = dense_key_range(p, r, b, pos);     // pos: row index of the row's first key
        j1 = n < jend ? n : jend;
    }
    // the same in every lane; taken from lane 0 so the tile loop's exits are uniform
    // branches and every trip of it starts with the same loads in flight
    const int nb = __builtin_amdgcn_readfirstlane(j1 > j0 ? (int)((j1 - j0 + kTileKeys - 1) / kTileKeys) : 0);
    const int64_t vdelta = LIST == KEYS_LATENT  ? 0
                           : LIST == KEYS_DENSE ? static_cast<const char *>(p.dense_v) - static_cast<const char *>(p.dense_k)
                                                : (int64_t)p.kv.plane_stride_b;
    const char *dummy = qrow0;                   // a readable row for absent keys

    float m = kNoKey, lsum = 0.f;                // head li (shared by the 4 lanes of li)
    f32x4_t acc[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t)
        acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // with a positive scale the maximum of the scaled scores is the scaled maximum, so
    // the scale is applied once to the maximum and folded into the exponent's FMA
    const bool fold = p.scale_log2 > 0.f;

    // Each key's K and V row addresses go to the wavefront's LDS; the rows are then
    // loaded row-contiguous: load instruction i of a plane reads rows
    // i*KPI .. i*KPI + KPI-1, LPK lanes per row, every lane reading its row's addresses
    // back from LDS (all reads in flight at once, one wait).
    const int my_row = lane / LPK;              // row within a load instruction
    const int my_chunk = lane % LPK;            // 16-byte chunk within the row
    struct Pages { KeyPos k; int32_t slot; uint32_t page; };
    struct Rows { u32x4 k[NI], v[NI]; uint32_t present; };
    const int chunk_b = my_chunk * 16;

    auto load_pages = [&](int batch, const Entries &E, Pages &P) {
        const int64_t jj = key_index(batch);
        P.k = key_pos<LIST>(p, pos, jj, E.raw, jj < j1);
        if constexpr (LIST == KEYS_DENSE) {
            P.page = 0;                            // dense: no page table
            P.slot = 0;
        } else {
            P.page = *page_entry_ptr<LIST>(p, b, P.k, P.slot);
        }
    };
    auto load_rows = [&](const Pages &P, Rows &R) {
        bool ok;
        const char *a = row_address<EB, LIST>(p, P.k, P.page, P.slot, g, dummy, ok);
        R.present = (uint32_t)(__ballot(ok) & 0xffffffffull);
        // an absent key reads the q row for both planes (its weight is zero). The
        // previous tile's reads of these slots came earlier in this wavefront's LDS order.
        // Lanes l and l + 32 walk the same key and store the same pair (no branch). The
        // empty asm statements tell the compiler that other lanes change these slots:
        // without them it may take a lane to read back what it read the previous time
        // (nothing it stored changed them) and reuse that load's rows.
        asm volatile("" ::: "memory");
        s_rows[kl] = u64x2{(uint64_t)(uintptr_t)a, (uint64_t)(uintptr_t)(ok ? a + vdelta : dummy)};
        asm volatile("" ::: "memory");
        u64x2 e[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i)
            e[i] = s_rows[i * KPI + my_row];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            R.k[i] = ldg16(reinterpret_cast<const char *>((uintptr_t)e[i].x) + chunk_b);
            R.v[i] = ldg16(reinterpret_cast<const char *>((uintptr_t)e[i].y) + chunk_b);
        }
    };
    uint32_t present = 0u;                       // keys present in the staged tile
    // rows -> the wavefront's LDS tiles (V widened to bf16); LDS operations of one
    // wavefront execute in order, the empty asm statements keep the compiler from
    // moving the accesses across each other (the previous tile's reads come first)
    auto stage = [&](const Rows &R) {
        present = R.present;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = i * KPI + my_row;
            *reinterpret_cast<u32x4 *>(s_k + row * KROWB + my_chunk * 16) = R.k[i];
            if constexpr (DT == QSA_BF16) {
                *reinterpret_cast<u32x4 *>(s_v + row * VROW + my_chunk * 8) = R.v[i];
            } else {
                *reinterpret_cast<u32x4 *>(s_v + row * VROW + my_chunk * 16) =
                    e4m3x8_to_bf16x8(u32x2{R.v[i][0], R.v[i][1]});
                *reinterpret_cast<u32x4 *>(s_v + row * VROW + my_chunk * 16 + 8) =
                    e4m3x8_to_bf16x8(u32x2{R.v[i][2], R.v[i][3]});
            }
        }
        asm volatile("" ::: "memory");
    };
    auto compute = [&]() {
        // S^T (two 16-key halves); A = 8 dims of key 16h + i from the K tile
        f32x4_t st[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            st[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const char *kp = s_k + (16 * h + li) * KROWB + (32 * c + 8 * lq) * EB;
                if constexpr (DT == QSA_BF16)
                    st[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const u32x4 *>(kp)),
                                                                    as_bf16x8(qf[c]), st[h], 0, 0, 0);
                else
                    st[h] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
                        as_long(*reinterpret_cast<const u32x2 *>(kp)), as_long(qf[c]), st[h], 0, 0, 0);
            }
        }
        // scores (log2 domain once scaled), absent keys (only in a tile that is not full) at -inf
        float sc[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[h][i] = fold ? st[h][i] : st[h][i] * p.scale_log2;
        if (present != 0xffffffffu) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sc[h][i] = (present >> (16 * h + 4 * lq + i)) & 1u ? sc[h][i] : kNegInf;
        }
        float mx = score_max(score_max(score_max(sc[0][0], sc[0][1]), score_max(sc[0][2], sc[0][3])),
                         score_max(score_max(sc[1][0], sc[1][1]), score_max(sc[1][2], sc[1][3])));
        mx = xor32_max(xor16_max(mx));
        mx = score_max(fold ? mx * p.scale_log2 : mx, m);
        if (__any(mx > m + kSlack)) {
            const float alpha = __builtin_amdgcn_exp2f(m - mx);
            lsum *= alpha;
#pragma unroll
            for (int t = 0; t < NDT; ++t)
                acc[t] *= alpha;
            m = mx;
        }
        float w[2][4];
        const float sl = fold ? p.scale_log2 : 1.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[h][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[h][i], sl, -m));
                lsum += w[h][i];
            }
        // P^T as the B operand: k-slot t < 4 is key 4q + t, t >= 4 is key 16 + 4q + t - 4
        const u32x4 pb = {pack_bf16x2(w[0][0], w[0][1]), pack_bf16x2(w[0][2], w[0][3]),
                          pack_bf16x2(w[1][0], w[1][1]), pack_bf16x2(w[1][2], w[1][3])};
        // V^T as the A operand via transposing LDS reads: source lane (q, 4j + e4) reads
        // 4 dims of key kb + j, and lane (q, i) receives dim i of keys kb .. kb + 3
        const int jr = li >> 2, qd = li & 3;
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
            const int col = 16 * t + 4 * qd;
            const s16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(s_v + (4 * lq + jr) * VROW + col));
            const s16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4 *)(s_v + (16 + 4 * lq + jr) * VROW + col));
            u32x4 av;
            __builtin_memcpy(&av, &a0, 8);
            __builtin_memcpy(reinterpret_cast<char *>(&av) + 8, &a1, 8);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(pb), acc[t], 0, 0, 0);
        }
        asm volatile("" ::: "memory");
    };

    // One register set of rows: tile i is copied to the wavefront's LDS tile as soon as
    // it has arrived, then tile i + 1's rows are issued into the same registers and
    // tile i is computed from LDS while they are in flight. Every trip starts with
    // entries i + 2, pages i + 1 and rows i in flight.
    if (nb > 0) {
        Pages P0, P1;
        Rows R;
        load_pages(0, E0, P0);
        load_entries(2, E0);
        load_pages(1, E1, P1);
        load_rows(P0, R);
        for (int i = 0;; i += 2) {
            stage(R);                            // rows i
            load_rows(P1, R);                    // rows i + 1
            load_entries(i + 3, E1);
            load_pages(i + 2, E0, P0);
            compute();                           // tile i
            if (i + 1 >= nb)
                break;
            stage(R);                            // rows i + 1
            load_rows(P0, R);                    // rows i + 2
            load_entries(i + 4, E0);
            load_pages(i + 3, E1, P1);
            compute();                           // tile i + 1
            if (i + 2 >= nb)
                break;
        }
    }

    // Per-head sum over the four lanes of each head. Lane (i, q) holds dims 16t + 4q ..
    // 16t + 4q + 3 of head i, so a direct store would write 32- or 64-byte pieces of up
    // to 16 rows per instruction; the values pass through this wavefront's own LDS
    // region (free after its last tile; 16 head slots x D bytes, padded by 16) so that
    // every store writes whole 16-byte chunks of one row, D bytes of a head per pass
    // (two passes of bf16, four of fp32).
    lsum = xor32_sum(xor16_sum(lsum));
    {
        constexpr int RS = D + 16;              // staging bytes per head slot
        constexpr int CPR = D / 16;             // 16-byte chunks per head and pass
        static_assert(16 * RS <= kWaveLds, "the staging rows fit the wavefront's LDS region");
        static_assert(D % 64 == 0, "whole wavefront stores");
        char *stage = s_k;
        const int64_t head0 = (int64_t)g * G;   // this kv head's first q head
        float scale = 1.f;
        if (S == 1 && li < G)
            scale = final_factor(p, head0 + li, m, lsum);
        auto emit = [&](auto ob, char *dst0, int64_t row_bytes) {
            constexpr int OB = decltype(ob)::value;
            constexpr int PT = D / OB / 16;     // MFMA tiles per pass
#pragma unroll
            for (int pass = 0; pass < OB; ++pass) {
                asm volatile("" ::: "memory");  // after the last tile's reads of this region
#pragma unroll
                for (int tl = 0; tl < PT; ++tl) {
                    const f32x4_t v = acc[pass * PT + tl] * scale;
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
                for (int j = 0; j < D / 64; ++j) {
                    const int c = j * 64 + lane;
                    const int hh = c / CPR, q = c % CPR;
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + hh * RS + q * 16);
                    if (hh < G)
                        *reinterpret_cast<u32x4 *>(dst0 + (int64_t)hh * row_bytes + pass * D + q * 16) = v;
                }
            }
        };
        if (S == 1) {
            const int eb = p.out_dtype == QSA_BF16 ? 2 : 4;
            char *dst0 = static_cast<char *>(p.out) + (r * p.num_q_heads + head0) * (int64_t)D * eb;
            if (p.out_dtype == QSA_BF16)
                emit(std::integral_constant<int, 2>{}, dst0, (int64_t)D * 2);
            else
                emit(std::integral_constant<int, 4>{}, dst0, (int64_t)D * 4);
        } else {
            const int64_t srh0 = (int64_t)s * p.total_q * p.num_q_heads + r * p.num_q_heads + head0;
            emit(std::integral_constant<int, 4>{}, reinterpret_cast<char *>(p.ws_acc + srh0 * D), (int64_t)D * 4);
            if (lq == 0 && li < G) {
                p.ws_ml[(srh0 + li) * 2] = m;
                p.ws_ml[(srh0 + li) * 2 + 1] = lsum;
            }
        }
    }
}

template <int DT, int D, int LIST>
int launch_mfma(const GatherParams &p, void *stream)
{
    const int waves = p.waves < kMfmaMaxWaves ? p.waves : kMfmaMaxWaves;
    const int64_t items = p.total_q * (int64_t)p.num_kv_heads * p.num_splits;
    const int64_t grid = (items + waves - 1) / waves;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gather_mfma_kernel<DT, D, LIST>), dim3((unsigned)grid), dim3(64 * waves), 0,
                       static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

template <int LIST>
int launch_mfma_t(const GatherParams &p, void *stream)
{
    if (p.dtype == QSA_BF16) {
        switch (p.head_dim) {
        case 64: return launch_mfma<QSA_BF16, 64, LIST>(p, stream);
        case 128: return launch_mfma<QSA_BF16, 128, LIST>(p, stream);
        case 256: return launch_mfma<QSA_BF16, 256, LIST>(p, stream);
        default: return (int)hipErrorInvalidValue;
        }
    }
    if (p.dtype == QSA_FP8_E4M3) {
        switch (p.head_dim) {
        case 64: return launch_mfma<QSA_FP8_E4M3, 64, LIST>(p, stream);
        case 128: return launch_mfma<QSA_FP8_E4M3, 128, LIST>(p, stream);
        case 256: return launch_mfma<QSA_FP8_E4M3, 256, LIST>(p, stream);
        default: return (int)hipErrorInvalidValue;
        }
    }
    return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_gather_mfma(const GatherParams &p, void *stream)
{
    switch (p.list_kind) {
    case KEYS_TOKEN_INDICES: return launch_mfma_t<KEYS_TOKEN_INDICES>(p, stream);
    case KEYS_BLOCKS: return launch_mfma_t<KEYS_BLOCKS>(p, stream);
    case KEYS_LATENT: return launch_mfma_t<KEYS_LATENT>(p, stream);
    case KEYS_DENSE: return launch_mfma_t<KEYS_DENSE>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace qsa
