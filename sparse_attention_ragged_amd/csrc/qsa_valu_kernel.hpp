// Gather-attention kernel on wavefront dot products (groups of 1, 2 or 4 query
// heads per kv head). Included by one translation unit per element type
// (qsa_valu_f32.hip, qsa_valu_bf16.hip, qsa_valu_e4m3.hip), so the instances build in parallel.
//
// One workgroup owns one (query row, kv head, split) and walks that split of the
// row's key list ("QSASparseAttentionRaggedPaged": token_indices up to counts;
// "Struct_msa_attention_ragged_paged": the positions of the listed blocks up to the
// row's position; "latent_sparse_attention_ragged_paged": window positions, then
// listed compressed entries). The per-team scoring, softmax fold and team merge are
// the shared core of qsa_valu_core.hpp.
//
//  * Head blocks: when all kv heads read the same keys (token-index and latent
//    lists), a workgroup covers a block of HB kv heads and the teams of a wavefront
//    are HB heads x (64/TL/HB) key slots. At HB = 8 (bf16, head_dim 128, 8 kv heads) a
//    wavefront reads a key's whole K block and V block (all heads, contiguous in the
//    page) with one request each, and the key's address is computed once per
//    wavefront. Key slots take keys j0 + b*NK*U + u*NK + slot (batch b, u < U, NK slots
//    per workgroup).
//  * Address staging: a workgroup walks its keys in chunks of kAddrPerThread keys
//    per thread. For a chunk, every thread loads the list entries of its keys (all at
//    once), then their page-table entries, and writes each key's row address (bit 0 =
//    present) to LDS; one barrier later the chunk's rows stream. Absent keys (past the
//    list, clipped, unused or outside the cache) read a harmless dummy row.
//  * Row pipeline (the pages' `unroll`, gathered keys in flight before any is
//    consumed): register sets of rows rotate, so that while batch b is folded into
//    the softmax state the rows of batch b+1 (and b+2, with three sets for groups of
//    1 or 2 heads) are in flight. The steady loop issues nothing but row loads, so
//    the in-order memory counter waits for exactly the oldest batch.
//  * Merge: teams of a wavefront merge with lane shuffles, wavefronts through LDS;
//    the result is the normalised output row (one split) or an (m, l, acc) partial
//    for the split-K combine kernel.
#pragma once

#include <atomic>
#include <type_traits>

#include "qsa_valu_core.hpp"

namespace qsa {

namespace {

constexpr int kMaxWaves = 8;
// Keys whose row addresses each thread stages in LDS per chunk (8 bytes each): 16,
// or 8 where fewer registers are left for the staging loads (the widened fp32 q rows
// of four e4m3 heads; the two-leaf address choice of latent lists).
constexpr int addr_per_thread(int dt, int g, int list)
{
    return (dt == QSA_FP8_E4M3 && g == 4) || list == KEYS_LATENT ? 8 : 16;
}

// NT: the K/V row loads are non-temporal (chosen by the planner for calls whose rows
// are read once: one query row per sequence)
template <int DT, int D, int G, int U, int LIST, bool NT>
__global__ void __launch_bounds__(64 * kMaxWaves) gather_valu_kernel(GatherParams p)
{
    using Core = ValuCore<DT, D, G, U>;
    // register sets of rows: three (two batches in flight while one is folded) where
    // the q rows and accumulators of the group leave room, else two
    constexpr int kRowSets = G <= 2 ? 3 : 2;
    constexpr int kAddrPerThread = addr_per_thread(DT, G, LIST);
    constexpr int EB = Core::EB;
    constexpr int EPC = Core::EPC;
    constexpr int CPL = Core::CPL;
    constexpr int TL = Core::TL;
    constexpr int TPW = Core::TPW;
    // LDS: the chunk's row addresses while streaming; afterwards the wavefronts' merge
    // ([NW][HB*G][2] then [NW][HB*G][D] fp32)
    extern __shared__ __attribute__((aligned(16))) float smem[];

    const int S = p.num_splits;
    const int HB = p.head_block;                 // kv heads of this workgroup, one team each
    uint32_t bid = blockIdx.x;                   // grid < 2^31 (checked by the launcher)
    const uint32_t nhb = (uint32_t)(p.num_kv_heads / HB);
    const int gb = (int)(bid % nhb);
    bid /= nhb;
    const int s = (int)(bid % (uint32_t)S);
    const int64_t r = bid / (uint32_t)S;

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int ln = tid % TL;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int NW = nthreads >> 6;
    const int tw = lane / TL;                    // team within the wavefront
    const int hh = tw % HB;                      // its kv head within the block
    const int ks = tw / HB;                      // its key slot within the wavefront
    const int KPW = TPW / HB;                    // key slots per wavefront
    const int g = gb * HB + hh;
    const int NK = NW * KPW;                     // key slots per workgroup

    // prologue: list length and the q rows go out together
    int64_t n = LIST == KEYS_DENSE ? 0 : key_list_length(p, r);
    const char *qbase = static_cast<const char *>(p.q) + ((r * p.num_q_heads + (int64_t)g * G) * D) * EB;
    typename Core::Q q;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            q.raw[h][c] = ldg16(qbase + ((int64_t)h * D + Core::chunk_elem(c, ln)) * EB);
    int64_t pos = 0;
    const int b = find_seq_pos_wave(p.row_off,
                                    LIST == KEYS_TOKEN_INDICES || LIST == KEYS_DENSE ? nullptr : p.cache_lengths,
                                    p.batch, (uint32_t)r, pos);
    if constexpr (LIST == KEYS_DENSE)
        n = dense_key_range(p, r, b, pos);     // pos: row index of the row's first key
    const int64_t j0 = (int64_t)s * p.split_keys;
    const int64_t jend = j0 + p.split_keys;
    const int64_t j1 = n < jend ? n : jend;
    const int per_batch = NK * U;
    const int64_t vdelta = LIST == KEYS_LATENT  ? 0
                           : LIST == KEYS_DENSE ? static_cast<const char *>(p.dense_v) - static_cast<const char *>(p.dense_k)
                                                : (int64_t)p.kv.plane_stride_b;
    const char *dummy = qbase;                   // a readable row for absent keys
    // the team's kv head within a key's row (the staged address is the head-0 row)
    const int64_t head_off = LIST == KEYS_LATENT ? 0 : (int64_t)g * D * EB;
    // list entries are per kv head only for block lists, which run one kv head per
    // workgroup (head_block 1)
    const int g_list = gb * HB;

    Core::widen_q(q);
    Core st;
    st.reset();

    uint64_t *s_addr = reinterpret_cast<uint64_t *>(smem);   // [chunk]: row address | present
    const int chunk = kAddrPerThread * nthreads;
    using Rows = typename Core::Rows;

    for (int64_t c0 = j0; c0 < j1; c0 += chunk) {
        const int cn = (int)(j1 - c0 < chunk ? j1 - c0 : chunk);
        // ---- stage this chunk's row addresses in LDS
        lds_barrier();                           // every wavefront is done with the previous chunk's
        {
            int32_t raw[kAddrPerThread];
#pragma unroll
            for (int k = 0; k < kAddrPerThread; ++k) {
                const int t = tid + k * nthreads;
                const int64_t jj = c0 + t;
                if constexpr (LIST == KEYS_DENSE)
                    raw[k] = 0;                  // dense: the key is its index, nothing to load
                else
                    raw[k] = *entry_ptr<LIST>(p, r, g_list, jj, t < cn);
            }
            KeyPos kp[kAddrPerThread];
            int32_t slot[kAddrPerThread];
            uint32_t page[kAddrPerThread];
#pragma unroll
            for (int k = 0; k < kAddrPerThread; ++k) {
                const int t = tid + k * nthreads;
                kp[k] = key_pos<LIST>(p, pos, c0 + t, raw[k], t < cn);
                if constexpr (LIST == KEYS_DENSE) {
                    page[k] = 0;                 // dense: no page table
                    slot[k] = 0;
                } else {
                    page[k] = *page_entry_ptr<LIST>(p, b, kp[k], slot[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < kAddrPerThread; ++k) {
                const int t = tid + k * nthreads;
                if (t < cn) {
                    bool ok;
                    const char *a = row_base<EB, LIST>(p, kp[k], page[k], slot[k], ok);
                    s_addr[t] = ok ? (reinterpret_cast<uint64_t>(a) | 1u) : 0u;
                }
            }
        }
        lds_barrier();

        // ---- stream the chunk's rows: batches b+1 and b+2 in flight while b is folded
        const int nb = (cn + per_batch - 1) / per_batch;
        auto issue = [&](int batch, Rows &R) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = batch * per_batch + u * NK + wave * KPW + ks;
                const uint64_t e = s_addr[t < cn ? t : cn - 1];
                const bool ok = t < cn && (e & 1u);
                const char *a = ok ? reinterpret_cast<const char *>(e & ~(uint64_t)15) + head_off : dummy;
                R.ok[u] = ok;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const char *ka = a + (int64_t)Core::chunk_elem(c, ln) * EB;
                    R.k[u][c] = NT ? ldg16_nt(ka) : ldg16(ka);
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const char *va = (ok ? a + vdelta : dummy) + (int64_t)Core::chunk_elem(c, ln) * EB;
                    R.v[u][c] = NT ? ldg16_nt(va) : ldg16(va);
                }
            }
            // keep the fold of the previous batch below these loads: hoisted above them it
            // would wait for that batch's rows before the next batch is issued
            __builtin_amdgcn_sched_barrier(0);
        };
        // Whole loop bodies only (a batch past the end holds no key and folds nothing),
        // so that the loop is entered and repeated with the same loads in flight.
        if constexpr (kRowSets == 3) {
            Rows R0, R1, R2;
            issue(0, R0);
            issue(1, R1);
            for (int i = 0; i < nb; i += 3) {
                issue(i + 2, R2);
                st.consume(R0, q, p.scale_log2);
                issue(i + 3, R0);
                st.consume(R1, q, p.scale_log2);
                issue(i + 4, R1);
                st.consume(R2, q, p.scale_log2);
            }
        } else {
            Rows R0, R1;
            issue(0, R0);
            for (int i = 0; i < nb; i += 2) {
                issue(i + 1, R1);
                st.consume(R0, q, p.scale_log2);
                issue(i + 2, R0);
                st.consume(R1, q, p.scale_log2);
            }
        }
        // (the loads of the batches past the chunk's end stay in flight: they read the
        // dummy row and are waited for with the next chunk's entries or at the end)
    }

    // merge the key slots of this wavefront (teams of the same kv head sit TL*HB
    // lanes apart)
    st.merge_teams(TL * HB);

    // merge the wavefronts through LDS (over the address chunk: every wavefront must be
    // done reading it): the key-slot-0 team of each kv head writes its state
    lds_barrier();
    const int HG = HB * G;                       // q heads of the workgroup
    float *s_ml = smem;                          // [NW][HG][2]
    float *s_acc = smem + ((NW * HG * 2 + 3) & ~3);   // [NW][HG][D], 16-byte aligned
    if (ks == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const int hq = hh * G + h;
            if (ln == 0) {
                s_ml[(wave * HG + hq) * 2] = st.m[h];
                s_ml[(wave * HG + hq) * 2 + 1] = st.l[h];
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int e = 0; e < EPC; e += 4)
                    *reinterpret_cast<float4 *>(&s_acc[(wave * HG + hq) * D + Core::chunk_elem(c, ln) + e]) =
                        make_float4(st.acc[h][c * EPC + e], st.acc[h][c * EPC + e + 1], st.acc[h][c * EPC + e + 2],
                                    st.acc[h][c * EPC + e + 3]);
        }
    }
    lds_barrier();
    // each thread finishes two adjacent outputs
    for (int idx = tid; idx < HG * D / 2; idx += nthreads) {
        const int hq = (2 * idx) / D;
        const int d = 2 * idx - hq * D;
        float M = kNoKey;
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, s_ml[(w * HG + hq) * 2]);
        float L = 0.f, A0 = 0.f, A1 = 0.f;
        for (int w = 0; w < NW; ++w) {
            const float c = __builtin_amdgcn_exp2f(s_ml[(w * HG + hq) * 2] - M);
            const float2 a = *reinterpret_cast<const float2 *>(&s_acc[(w * HG + hq) * D + d]);
            L += c * s_ml[(w * HG + hq) * 2 + 1];
            A0 += c * a.x;
            A1 += c * a.y;
        }
        const int64_t head = (int64_t)gb * HG + hq;
        const int64_t rh = r * p.num_q_heads + head;
        if (S == 1) {
            const float f = final_factor(p, head, M, L);
            store_out2(p.out, p.out_dtype, rh * D + d, A0 * f, A1 * f);
        } else {
            const int64_t srh = (int64_t)s * p.total_q * p.num_q_heads + rh;
            *reinterpret_cast<float2 *>(&p.ws_acc[srh * D + d]) = make_float2(A0, A1);
            if (d == 0) {
                p.ws_ml[srh * 2] = M;
                p.ws_ml[srh * 2 + 1] = L;
            }
        }
    }
}

template <int DT, int D, int G, int U, int LIST, bool NT>
int launch_valu_nt(const GatherParams &p, void *stream)
{
    const int64_t grid = p.total_q * (int64_t)(p.num_kv_heads / p.head_block) * p.num_splits;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    // LDS of the cross-wavefront merge: (reference, sum) and D partial outputs per q head
    const size_t hg = (size_t)p.waves * p.head_block * G;
    const size_t merge = (((2 * hg + 3) & ~(size_t)3) + hg * D) * sizeof(float);
    const size_t addrs = (size_t)addr_per_thread(DT, G, LIST) * 64 * p.waves * sizeof(uint64_t);
    const size_t lds = merge > addrs ? merge : addrs;
    // allow more than the default dynamic LDS, once per device
    static std::atomic<uint64_t> raised{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        dev = 63;
    if (!(raised.load() >> dev & 1u)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gather_valu_kernel<DT, D, G, U, LIST, NT>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess)
            return (int)e;
        raised.fetch_or(uint64_t(1) << dev);
    }
    hipLaunchKernelGGL((gather_valu_kernel<DT, D, G, U, LIST, NT>), dim3((unsigned)grid), dim3(64 * p.waves),
                       lds, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

// non-temporal row loads only exist for the index lists (dense and latent rows are
// shared by neighbouring rows)
template <int DT, int D, int G, int U, int LIST>
int launch_valu(const GatherParams &p, void *stream)
{
    if constexpr (LIST == KEYS_TOKEN_INDICES || LIST == KEYS_BLOCKS) {
        if (p.stream_rows)
            return launch_valu_nt<DT, D, G, U, LIST, true>(p, stream);
    }
    return launch_valu_nt<DT, D, G, U, LIST, false>(p, stream);
}

// Two keys per team per batch: with two 16-byte chunks per lane that keeps as many
// bytes in flight as four one-chunk keys, and the register sets of both batches stay
// within the 256 VGPRs a wavefront has at two wavefronts per SIMD. (`unroll` is
// accepted for compatibility of launch options and does not change the kernel.)
template <int DT, int D, int G, int LIST>
int launch_valu_u(const GatherParams &p, void *stream)
{
    return launch_valu<DT, D, G, 2, LIST>(p, stream);
}

template <int DT, int D, int LIST>
int launch_valu_g(const GatherParams &p, void *stream)
{
    switch (p.group) {
    case 1: return launch_valu_u<DT, D, 1, LIST>(p, stream);
    case 2: return launch_valu_u<DT, D, 2, LIST>(p, stream);
    case 4: return launch_valu_u<DT, D, 4, LIST>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

template <int DT, int LIST>
int launch_valu_d(const GatherParams &p, void *stream)
{
    switch (p.head_dim) {
    case 64: return launch_valu_g<DT, 64, LIST>(p, stream);
    case 128: return launch_valu_g<DT, 128, LIST>(p, stream);
    case 256: return launch_valu_g<DT, 256, LIST>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

// every list kind of one element type
template <int DT>
int launch_valu_lists(const GatherParams &p, void *stream)
{
    switch (p.list_kind) {
    case KEYS_TOKEN_INDICES: return launch_valu_d<DT, KEYS_TOKEN_INDICES>(p, stream);
    case KEYS_BLOCKS: return launch_valu_d<DT, KEYS_BLOCKS>(p, stream);
    case KEYS_LATENT: return launch_valu_d<DT, KEYS_LATENT>(p, stream);
    case KEYS_DENSE: return launch_valu_d<DT, KEYS_DENSE>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace qsa
