// Latent gather-attention on matrix cores for wide head groups ("latent_sparse_attention_
// ragged_paged": one latent head whose row is both key and value, many query heads).
//
// One workgroup owns one (query row, split): 64 query heads in four tiles of 16 (heads
// past the group compute on zero queries and are not stored), keys 32 at a time. Its
// eight wavefronts take two roles, one of each per SIMD:
//
//  * score wavefront s (heads 16s..16s+15) computes, on 16x16x32 MFMAs,
//    S^T = X . Q^T (A: 8 dims of a key from the LDS key tile, B: the heads' q rows,
//    held in VGPRs), and runs the online softmax for its heads in the log2 domain
//    (lazy rescale), leaving P (bf16, already in the MFMA operand layout) and the
//    rescale factors in LDS;
//  * value wavefront s accumulates O^T += X^T P^T for the same heads one tile later
//    (A: transposing LDS reads of the key tile, B: P from LDS), and the sum of the
//    weights with one more MFMA whose A operand is all ones, and owns their output
//    rows.
//
// The value wavefronts also load: each walks its share of the keys of the split
// (window positions, then listed compressed entries) through the three-stage address
// pipeline and writes its chunks of their latent rows into an LDS key tile. Per tile:
// the value wavefronts store tile t+1 and issue loads, then score wavefronts score
// tile t while value wavefronts accumulate tile t-1; one barrier, which waits only
// for LDS traffic, ends the step (three LDS key tiles, two P buffers). The score
// step is the longer one, so leaving the loading to the value wavefronts shortens
// the step (measured at D 512: the score wavefronts' share of the loading sat on the
// critical path). The vector-memory counter retires loads in issue order, so the
// three address stages run DEPTH, 2*DEPTH and 3*DEPTH tiles ahead (rows, page-table
// entries, list entries) and no step waits for anything newer than the tile it
// stores; DEPTH is one tile, all the value wavefronts' registers allow next to their
// accumulators. LDS operand reads are software-pipelined a few MFMAs ahead. The per-head
// sink logit joins the denominator once, at the final normalisation (here with one
// split, in the combine kernel otherwise).
#include "qsa_device.hpp"

#include <type_traits>

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

constexpr int kWaves = 4;             // head tiles (64 heads); one score + one value wavefront each
static_assert(16 * kWaves == kWideMaxGroup, "the host-side support check assumes 64 heads per workgroup");
constexpr int kWTile = 32;            // keys per tile
constexpr int kDepth = 1;             // tiles of rows in flight (in the value wavefronts' registers)
constexpr int kXBufs = 3;             // LDS key tiles: being written, scored, accumulated
constexpr int kUnroll = 6;            // steps per loop trip: register slots and LDS tiles static
constexpr float kWSlack = 8.0f;
constexpr int kPrefetch = 4;          // MFMA steps of LDS operand reads kept in flight
constexpr int kWThreads = 64 * 2 * kWaves;

__device__ __forceinline__ bf16x8_t wide_bf16x8(u32x4 v)
{
    bf16x8_t r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

template <int D>
__global__ void __launch_bounds__(kWThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gather_mfma_wide_kernel(GatherParams p)
{
    constexpr int EB = 2;                       // bf16
    constexpr int NC = D / 32;
    constexpr int NDT = D / 16;
    // LDS row (bf16 elements): 32 bytes of padding keep both the 16-byte row reads of
    // the score step and the transposing reads of the value step free of bank conflicts
    constexpr int ROW = D + 16;
    constexpr int CHUNKS = D * EB / 16;         // 16-byte chunks of one row
    static_assert(D % 32 == 0, "head_dim must be a multiple of 32");
    __shared__ __attribute__((aligned(16))) uint16_t s_x[kXBufs][kWTile * ROW];
    __shared__ __attribute__((aligned(16))) u32x4 s_p[2][kWaves][64];   // P^T operands
    __shared__ float s_alpha[2][kWaves][16];    // rescale factor per head (when flagged)
    __shared__ uint32_t s_flag[2][kWaves];      // 1: the value wavefront rescales before adding
    __shared__ uint32_t s_ok[kXBufs][2 * kWaves];   // presence bits of each wavefront's keys
    __shared__ float s_m[kWaves][16];           // final reference per head

    // loading layout (value wavefronts only): TPK threads per key, each loading CPT
    // chunks (chunk u*TPK + sub); value wavefront w stages keys KPW*w .. KPW*w + KPW-1
    constexpr int kLoaders = 64 * kWaves;
    constexpr int TPK = kLoaders / kWTile;
    constexpr int CPT = CHUNKS / TPK;
    constexpr int KPW = 64 / TPK;
    static_assert(CHUNKS % TPK == 0, "row chunks must split evenly over a key's threads");

    // rows before split_row0 run unsplit (one workgroup each, first in the grid); the
    // rest run num_splits ways
    const int64_t R0 = p.split_row0;
    const bool whole = (int64_t)blockIdx.x < R0;
    const int S = whole ? 1 : p.num_splits;
    const int64_t t_split = whole ? 0 : (int64_t)blockIdx.x - R0;
    const int s = (int)(t_split % S);
    const int64_t r = whole ? (int64_t)blockIdx.x : R0 + t_split / S;
    const int G = p.group;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int lq = lane >> 4;
    const int hw = wave % kWaves;               // head tile of this wavefront
    const int head = 16 * hw + li;              // within the group
    const bool head_real = head < G;

    const int64_t n = key_list_length(p, r);
    const int64_t j0 = (int64_t)s * p.split_keys;                 // 0 for an unsplit row
    const int64_t j1 = whole || n < j0 + p.split_keys ? n : j0 + p.split_keys;
    const int nb = j1 > j0 ? (int)((j1 - j0 + kWTile - 1) / kWTile) : 0;
    // steps: nb scores, then the value step of the last tile (the loop body is unrolled
    // so that register slots and LDS tiles stay static, and leaves after step nb)
    const int nsteps = nb > 0 ? nb + 1 : 0;
    const char *qrow0 = static_cast<const char *>(p.q) + (r * p.num_q_heads) * D * EB;

    const bool is_score = wave >= kWaves;
    // normalised output rows of this wavefront's heads (one split) or the split's partial
    auto finish = [&](float m, float lsum, const f32x4_t *acc, float sink_l2) {
        const int64_t gh = (int64_t)head;       // the single kv head: group = all q heads
        if (!head_real)
            return;
        const int64_t rh = r * p.num_q_heads + gh;
        if (S == 1) {
            float inv;
            if (p.sink) {                       // the sink logit, loaded at the start
                const float M2 = fmaxf(m, sink_l2);
                const float c = __builtin_amdgcn_exp2f(m - M2);
                const float L = lsum * c + __builtin_amdgcn_exp2f(sink_l2 - M2);
                inv = L > 0.f ? c / L : 0.f;
            } else {
                inv = lsum > 0.f ? 1.f / lsum : 0.f;
            }
#pragma unroll
            for (int t = 0; t < NDT; ++t)
                store_out4(p.out, p.out_dtype, rh * D + 16 * t + 4 * lq, acc[t] * inv);
        } else {
            const int64_t srh = ((int64_t)s * (p.total_q - R0) + (r - R0)) * p.num_q_heads + gh;
#pragma unroll
            for (int t = 0; t < NDT; ++t)
                *reinterpret_cast<f32x4_t *>(p.ws_acc + srh * D + 16 * t + 4 * lq) = acc[t];
            if (lq == 0) {
                p.ws_ml[srh * 2] = m;
                p.ws_ml[srh * 2 + 1] = lsum;
            }
        }
    };
    // The same, once every key tile is consumed: in the MFMA layout a lane holds four
    // positions of one head, so a direct store writes 32-byte pieces of 16 rows per
    // instruction (measured: about 7700 cycles for a 64-head row of D 512, most of a
    // workgroup's epilogue). Instead the values pass through this wavefront's own eight
    // rows of key tile 0 (16 heads x D bytes, rows padded by 16 bytes) so that every
    // store writes whole 16-byte chunks of one row, D bytes of a head per pass (two
    // passes of bf16, four of fp32).
    auto finish_staged = [&](float m, float lsum, const f32x4_t *acc, float sink_l2) {
        constexpr int RS = D + 16;              // bytes per head in the staging rows
        constexpr int CPR = D / 16;             // 16-byte chunks per head and pass
        char *stage = reinterpret_cast<char *>(s_x[0] + 8 * hw * ROW);
        float scale = 1.f;
        if (S == 1) {
            if (p.sink) {                       // the sink logit, loaded at the start
                const float M2 = fmaxf(m, sink_l2);
                const float c = __builtin_amdgcn_exp2f(m - M2);
                const float L = lsum * c + __builtin_amdgcn_exp2f(sink_l2 - M2);
                scale = L > 0.f ? c / L : 0.f;
            } else {
                scale = lsum > 0.f ? 1.f / lsum : 0.f;
            }
        }
        auto emit = [&](auto ob, char *dst0, int64_t row_bytes) {
            constexpr int OB = decltype(ob)::value;
            constexpr int PT = D / OB / 16;     // MFMA tiles per pass
#pragma unroll
            for (int pass = 0; pass < OB; ++pass) {
                asm volatile("" ::: "memory");
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
                    if (16 * hw + hh < G)
                        *reinterpret_cast<u32x4 *>(dst0 + (int64_t)hh * row_bytes + pass * D + q * 16) = v;
                }
            }
        };
        if (S == 1) {
            const int eb = p.out_dtype == QSA_BF16 ? 2 : 4;
            char *dst0 = static_cast<char *>(p.out) + (r * p.num_q_heads + 16 * hw) * (int64_t)D * eb;
            if (p.out_dtype == QSA_BF16)
                emit(std::integral_constant<int, 2>{}, dst0, (int64_t)D * 2);
            else
                emit(std::integral_constant<int, 4>{}, dst0, (int64_t)D * 4);
        } else {
            const int64_t srh0 = ((int64_t)s * (p.total_q - R0) + (r - R0)) * p.num_q_heads + 16 * hw;
            emit(std::integral_constant<int, 4>{}, reinterpret_cast<char *>(p.ws_acc + srh0 * D), (int64_t)D * 4);
            if (lq == 0 && head_real) {
                p.ws_ml[(srh0 + li) * 2] = m;
                p.ws_ml[(srh0 + li) * 2 + 1] = lsum;
            }
        }
    };
    if (nb == 0) {                              // no keys: zeros (or an empty partial)
        if (!is_score) {
            f32x4_t zero[NDT];
#pragma unroll
            for (int t = 0; t < NDT; ++t)
                zero[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            finish(kNoKey, 0.f, zero, kNegInf);
        }
        return;
    }
    {
        int b = 0;          // sequence and position: found after the first list entries left
        int64_t pos = 0;
        const char *dummy = qrow0;
        const int skey = tid / TPK;
        const int ssub = tid % TPK;

        struct Page { KeyPos k; int32_t slot; uint32_t page; };
        struct Rows { u32x4 x[CPT]; bool ok; };

        auto key_index = [&](int tile) -> int64_t { return j0 + (int64_t)tile * kWTile + skey; };
        auto load_entry = [&](int tile) -> int32_t {
            const int64_t jj = key_index(tile);
            return *entry_ptr<KEYS_LATENT>(p, r, 0, jj, jj < j1);
        };
        auto load_page = [&](int tile, int32_t raw, Page &P) {
            const int64_t jj = key_index(tile);
            P.k = key_pos<KEYS_LATENT>(p, pos, jj, raw, jj < j1);
            P.page = *page_entry_ptr<KEYS_LATENT>(p, b, P.k, P.slot);
        };
        auto load_rows = [&](const Page &P, Rows &R) {
            bool ok;
            const char *a = row_address<EB, KEYS_LATENT>(p, P.k, P.page, P.slot, 0, dummy, ok);
            R.ok = ok;
            const char *base = ok ? a : dummy;
#pragma unroll
            for (int u = 0; u < CPT; ++u)
                R.x[u] = ldg16(base + (int64_t)(u * TPK + ssub) * 16);
        };
        // rows -> LDS tile `buf`, presence bits -> s_ok[buf][wave]; visible after the next barrier
        auto store_rows = [&](const Rows &R, int buf) {
            uint16_t *row = s_x[buf] + skey * ROW;
#pragma unroll
            for (int u = 0; u < CPT; ++u)
                *reinterpret_cast<u32x4 *>(row + (u * TPK + ssub) * 8) = R.x[u];
            const unsigned long long bal = __ballot(R.ok);
            uint32_t bits = 0;
#pragma unroll
            for (int k = 0; k < KPW; ++k)
                bits |= (uint32_t)((bal >> (k * TPK)) & 1ull) << k;
            if (lane == 0)
                s_ok[buf][wave] = bits;
        };

        // `xb`: the LDS key tile holding `tile`, tile % 3 (a compile-time constant in the
        // unrolled steps)
        // the value wavefront also keeps the running sum of the weights, by an MFMA with an
        // all-ones A operand (every element of lsum is the sum over the keys, for head li,
        // of the same bf16-rounded weights that P.V uses)
        const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};   // bf16 1.0 pairs
        auto accumulate = [&](int tile, int xb, f32x4_t *acc, f32x4_t &lsum) {
            const int pb_buf = tile & 1;
            if (s_flag[pb_buf][hw]) {
                const float alpha = s_alpha[pb_buf][hw][li];
                lsum *= alpha;
#pragma unroll
                for (int t = 0; t < NDT; ++t)
                    acc[t] *= alpha;
            }
            const u32x4 pb = s_p[pb_buf][hw][lane];
            lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wide_bf16x8(ones), wide_bf16x8(pb), lsum, 0, 0, 0);
            const uint16_t *x = s_x[xb];
            const int jr = li >> 2, qd = li & 3;
            // A = X^T for 16 dims x 32 keys: two transposing reads (keys 4q..4q+3 and
            // 16+4q..16+4q+3 of dims 16t+4qd..+3)
            auto read_a = [&](int t) {
                const int col = 16 * t + 4 * qd;
                const s16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(x + (4 * lq + jr) * ROW + col));
                const s16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(x + (16 + 4 * lq + jr) * ROW + col));
                u32x4 av;
                __builtin_memcpy(&av, &a0, 8);
                __builtin_memcpy(reinterpret_cast<char *>(&av) + 8, &a1, 8);
                return av;
            };
            // software pipeline: the reads of step t+PF are issued before the MFMA of
            // step t (scheduling fences keep the order)
            u32x4 av[kPrefetch];
#pragma unroll
            for (int t = 0; t < kPrefetch; ++t)
                av[t] = read_a(t);
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const u32x4 a = av[t % kPrefetch];
                if (t + kPrefetch < NDT)
                    av[t % kPrefetch] = read_a(t + kPrefetch);
                __builtin_amdgcn_sched_barrier(0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wide_bf16x8(a), wide_bf16x8(pb), acc[t], 0, 0, 0);
            }
        };

        // with a positive scale the maximum of the scaled scores is the scaled maximum, so
        // the scale is applied once to the maximum and folded into the exponent's FMA
        const bool fold = p.scale_log2 > 0.f;
        auto score = [&](int tile, int xb, const u32x4 *qf, float &m) {
            const uint16_t *x = s_x[xb];
            uint32_t present = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                present |= s_ok[xb][w] << (w * KPW);
            // two chains per key half (even / odd 32-dim chunks) halve the MFMA dependency depth
            f32x4_t st[2], st2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                st[h] = st2[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // A = 16 keys x 32 dims of X (keys 16h + i), one 16-byte read per lane;
            // software-pipelined like the value step
            auto read_k = [&](int c, int h) {
                return *reinterpret_cast<const u32x4 *>(x + (16 * h + li) * ROW + 32 * c + 8 * lq);
            };
            u32x4 kf[kPrefetch][2];
#pragma unroll
            for (int c = 0; c < kPrefetch; ++c) {
                kf[c][0] = read_k(c, 0);
                kf[c][1] = read_k(c, 1);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 k0 = kf[c % kPrefetch][0], k1 = kf[c % kPrefetch][1];
                if (c + kPrefetch < NC) {
                    kf[c % kPrefetch][0] = read_k(c + kPrefetch, 0);
                    kf[c % kPrefetch][1] = read_k(c + kPrefetch, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x4_t *sa = c & 1 ? st2 : st;
                sa[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wide_bf16x8(k0), wide_bf16x8(qf[c]), sa[0], 0, 0, 0);
                sa[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wide_bf16x8(k1), wide_bf16x8(qf[c]), sa[1], 0, 0, 0);
            }
            st[0] += st2[0];
            st[1] += st2[1];
            float sc[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sc[h][i] = fold ? st[h][i] : st[h][i] * p.scale_log2;
            if (present != 0xffffffffu) {        // absent keys (only in a tile that is not full) at -inf
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
            const int pb_buf = tile & 1;
            uint32_t flag = 0;
            if (__any(mx > m + kWSlack)) {
                const float alpha = __builtin_amdgcn_exp2f(m - mx);
                m = mx;
                if (lq == 0)
                    s_alpha[pb_buf][hw][li] = alpha;
                flag = 1;
            }
            if (lane == 0)
                s_flag[pb_buf][hw] = flag;
            float w[2][4];
            const float sl = fold ? p.scale_log2 : 1.f;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[h][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[h][i], sl, -m));
            s_p[pb_buf][hw][lane] = u32x4{pack_bf16x2(w[0][0], w[0][1]), pack_bf16x2(w[0][2], w[0][3]),
                                          pack_bf16x2(w[1][0], w[1][1]), pack_bf16x2(w[1][2], w[1][3])};
        };

        // pipeline fill: list entries of tiles 0..3*DEPTH, page entries of 0..2*DEPTH,
        // rows of 0..DEPTH (issue order = retirement order)
        int32_t E[kDepth];
        Page P[kDepth];
        Rows R[kDepth];
        // the score wavefronts' q rows and the value wavefronts' sink logit are loaded
        // here, before the first barrier, so that their latency overlaps the dependent
        // chain (list entries -> sequence -> page entries -> rows) of the first tile
        // B operand of S^T: 8 dims of this lane's head per 32-dim chunk (zeros for padding heads)
        u32x4 qf[NC];
        float sink_l2 = kNegInf;
        if (is_score) {
            const char *qrow = qrow0 + (int64_t)(head_real ? head : 0) * D * EB;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 v = ldg16(qrow + (32 * c + 8 * lq) * EB);
                qf[c] = head_real ? v : u32x4{0, 0, 0, 0};
            }
        } else if (p.sink) {
            sink_l2 = p.sink[head_real ? head : 0] * 1.44269504088896340736f;
        }
        if (!is_score) {
            int32_t e_fill[3 * kDepth + 1];
#pragma unroll
            for (int j = 0; j <= 3 * kDepth; ++j)
                e_fill[j] = load_entry(j);
            b = find_seq_pos_wave(p.row_off, p.cache_lengths, p.batch, (uint32_t)r, pos);
            Page p_fill[2 * kDepth + 1];
#pragma unroll
            for (int j = 0; j <= 2 * kDepth; ++j)
                load_page(j, e_fill[j], p_fill[j]);
            Rows r0;
            load_rows(p_fill[0], r0);
#pragma unroll
            for (int j = 1; j <= kDepth; ++j)
                load_rows(p_fill[j], R[j % kDepth]);
            // steady-state registers before step t: R[j % DEPTH] holds the rows of tiles
            // t+1 .. t+DEPTH, P[j % DEPTH] the page entries of t+1+DEPTH .. t+2*DEPTH and
            // E[j % DEPTH] the list entries of t+1+2*DEPTH .. t+3*DEPTH
#pragma unroll
            for (int j = kDepth + 1; j <= 2 * kDepth; ++j)
                P[j % kDepth] = p_fill[j];
#pragma unroll
            for (int j = 2 * kDepth + 1; j <= 3 * kDepth; ++j)
                E[j % kDepth] = e_fill[j];
            store_rows(r0, 0);
        }
        lds_barrier();

        // the steps; each role runs its own copy of the loop so that only its own state
        // is live in it. A store past the last tile writes a tile buffer nobody reads.
        // Every wavefront of the workgroup leaves after the same step (nsteps is the
        // workgroup's), so all pass the same barriers.
        static_assert(kUnroll % kDepth == 0 && kUnroll % kXBufs == 0, "static slots need a common period");
        auto steps = [&](auto &&work) {
            for (int t = 0;; t += kUnroll) {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int tt = t + u;
                    const int k = (u + 1) % kDepth;  // register slot of tiles tt+1 (+ multiples of DEPTH)
                    if (!is_score) {
                        store_rows(R[k], (u + 1) % kXBufs);          // tile tt+1 -> LDS tile (tt+1) % 3
                        load_rows(P[k], R[k]);                       // rows of tt+1+DEPTH
                        load_page(tt + 1 + 2 * kDepth, E[k], P[k]);  // pages of tt+1+2*DEPTH
                        E[k] = load_entry(tt + 1 + 3 * kDepth);      // entries of tt+1+3*DEPTH
                    }
                    work(tt, u);
                    lds_barrier();
                    if (tt + 1 >= nsteps)
                        return;
                }
            }
        };
        if (is_score) {
            float m = kNoKey;
            steps([&](int tt, int u) {
                if (tt < nb)
                    score(tt, u % kXBufs, qf, m);
            });
            if (lq == 0)
                s_m[hw][li] = m;
            lds_barrier();
            return;
        }
        f32x4_t acc[NDT], lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NDT; ++t)
            acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        steps([&](int tt, int u) {
            if (tt >= 1 && tt <= nb)
                accumulate(tt - 1, (u + kXBufs - 1) % kXBufs, acc, lsum);
        });
        lds_barrier();                          // the score wavefronts' final reference; tiles consumed
        finish_staged(s_m[hw][li], lsum[0], acc, sink_l2);
    }
}

template <int D>
int launch_wide(const GatherParams &p, void *stream)
{
    const int64_t grid = p.split_row0 + (p.total_q - p.split_row0) * (int64_t)p.num_splits;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gather_mfma_wide_kernel<D>), dim3((unsigned)grid), dim3(kWThreads), 0,
                       static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

}  // namespace

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
