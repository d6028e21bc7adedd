// Gather-attention kernel on wavefront dot products (groups of 1, 2 or 4 query
// heads per kv head).
//
// One workgroup owns one (query row, kv head, split) and walks that split of the
// row's key list ("QSASparseAttentionRaggedPaged": token_indices up to counts;
// "Struct_msa_attention_ragged_paged": the positions of the listed blocks up to the
// row's position; "latent_sparse_attention_ragged_paged": window positions, then
// listed compressed entries).
//
//  * Key teams: a team of TL = rowbytes/16 lanes owns one key at a time; each lane
//    holds one 16-byte chunk of the key's K row and of its V row. Teams take keys
//    j0 + b*NT*U + u*NT + team (batch b, slot u < U).
//  * Address pipeline (the pages' `unroll` keys in flight, and more): while batch b
//    is folded into the softmax state, the K/V rows of batch b+1 are in flight, the
//    page-table entries of batch b+2 and the list entries of batch b+3. Every stage
//    issues one load per key on every path (dummies for absent keys), so the compiler
//    waits for exactly the oldest batch. There is no staging phase and no barrier
//    before the first K/V load: a workgroup reaches full speed after three memory
//    latencies.
//  * Scores: per head, a lane's partial dot product (packed bf16 dot instruction on
//    the raw q and K words; fp32 FMAs otherwise) is summed over the team with DPP,
//    scaled into the log2 domain, and folded into a running (reference, sum, acc)
//    state in fp32. The reference only moves when a score exceeds it by more than
//    2^8 (then the whole wavefront rescales), so most batches skip the rescale.
//  * Merge: teams of a wavefront merge with lane shuffles, wavefronts through LDS;
//    the result is the normalised output row (one split) or an (m, l, acc) partial
//    for the split-K combine kernel.
#include "qsa_device.hpp"

namespace qsa {

namespace {

constexpr int kMaxWaves = 8;
constexpr float kRescaleSlack = 8.0f;   // log2 units: weights stay <= 2^8

template <int DT, int D, int G, int U, int LIST>
__global__ void __launch_bounds__(64 * kMaxWaves) gather_valu_kernel(GatherParams p)
{
    constexpr int EB = Elem<DT>::bytes;
    constexpr int ROWB = D * EB;                 // bytes of one K (or V) row
    constexpr int TL = ROWB / 16;                // lanes per key team
    constexpr int EPL = 16 / EB;                 // elements per lane
    static_assert(TL >= 2 && TL <= 64 && 64 % TL == 0, "unsupported head_dim for this dtype");
    __shared__ __attribute__((aligned(16))) float smem[kMaxWaves * G * (D + 2)];

    const int S = p.num_splits;
    const int Hkv = p.num_kv_heads;
    int64_t bid = blockIdx.x;
    const int g = (int)(bid % Hkv);
    bid /= Hkv;
    const int s = (int)(bid % S);
    const int64_t r = bid / S;

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int team = tid / TL;
    const int ln = tid % TL;
    const int NT = nthreads / TL;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int NW = nthreads >> 6;

    // prologue: list length, sequence and the q rows go out together
    const int64_t n = key_list_length(p, r);
    const char *qbase = static_cast<const char *>(p.q) + ((r * p.num_q_heads + (int64_t)g * G) * D) * EB;
    u32x4 qraw[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        qraw[h] = ldg16(qbase + ((int64_t)h * D + ln * EPL) * EB);
    const int b = find_seq_wave(p.row_off, p.batch, (uint32_t)r);
    int64_t pos = 0;
    if constexpr (LIST != KEYS_TOKEN_INDICES)
        pos = (int64_t)p.cache_lengths[b] + (r - (int64_t)p.row_off[b]);
    const int64_t j0 = (int64_t)s * p.split_keys;
    const int64_t j1 = n < j0 + p.split_keys ? n : j0 + p.split_keys;
    const int64_t per_batch = (int64_t)NT * U;
    const int nb = j1 > j0 ? (int)((j1 - j0 + per_batch - 1) / per_batch) : 0;
    const int64_t vdelta = LIST == KEYS_LATENT ? 0 : p.kv.plane_stride * EB;
    const char *dummy = qbase + (int64_t)ln * 16;   // a readable row for absent keys

    float qf[G][DT == QSA_BF16 ? 1 : EPL];
    if constexpr (DT != QSA_BF16) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (DT == QSA_F32)
                    qf[h][i] = __uint_as_float(qraw[h][i]);
                else
                    e4m3x4_to_f32(qraw[h][i], &qf[h][4 * i]);
            }
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNoKey;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[h][e] = 0.f;
    }

    // ---- pipeline stages (each issues exactly one load per key on every path)
    struct Entries { int32_t raw[U]; };
    struct Pages { KeyPos k[U]; int32_t slot[U]; uint32_t page[U]; };
    struct Rows { u32x4 k[U], v[U]; bool ok[U]; };

    auto key_index = [&](int batch, int u) -> int64_t { return j0 + batch * per_batch + u * NT + team; };
    auto load_entries = [&](int batch, Entries &E) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t jj = key_index(batch, u);
            E.raw[u] = *entry_ptr<LIST>(p, r, g, jj, jj < j1);
        }
    };
    auto load_pages = [&](int batch, const Entries &E, Pages &P) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t jj = key_index(batch, u);
            P.k[u] = key_pos<LIST>(p, pos, jj, E.raw[u], jj < j1);
            P.page[u] = *page_entry_ptr<LIST>(p, b, P.k[u], P.slot[u]);
        }
    };
    auto load_rows = [&](const Pages &P, Rows &R) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bool ok;
            const char *a = row_address<EB, LIST>(p, P.k[u], P.page[u], P.slot[u], g, dummy, ok);
            R.ok[u] = ok;
            R.k[u] = ldg16(ok ? a + ln * 16 : dummy);
            R.v[u] = ldg16(ok ? a + vdelta + ln * 16 : dummy);
        }
    };
    auto consume = [&](const Rows &R) {
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[DT == QSA_BF16 ? 1 : EPL];
            if constexpr (DT != QSA_BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (DT == QSA_F32)
                        kf[i] = __uint_as_float(R.k[u][i]);
                    else
                        e4m3x4_to_f32(R.k[u][i], &kf[4 * i]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
                if constexpr (DT == QSA_BF16) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qraw[h][i]), as_bf16x2(R.k[u][i]), d,
                                                            false);
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        d = fmaf(qf[h][e], kf[e], d);
                }
                d = team_sum<TL>(d) * p.scale_log2;
                sc[u][h] = R.ok[u] ? d : kNegInf;
            }
        }
        // lazy rescale of the running state
        float mx[G];
        bool need = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            mx[h] = m[h];
#pragma unroll
            for (int u = 0; u < U; ++u)
                mx[h] = fmaxf(mx[h], sc[u][h]);
            need |= mx[h] > m[h] + kRescaleSlack;
        }
        if (__any(need)) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float alpha = __builtin_amdgcn_exp2f(m[h] - mx[h]);
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[h][e] *= alpha;
                m[h] = mx[h];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (DT == QSA_F32) {
                    vf[i] = __uint_as_float(R.v[u][i]);
                } else if constexpr (DT == QSA_BF16) {
                    vf[2 * i] = bf16_lo(R.v[u][i]);
                    vf[2 * i + 1] = bf16_hi(R.v[u][i]);
                } else {
                    e4m3x4_to_f32(R.v[u][i], &vf[4 * i]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float w = __builtin_amdgcn_exp2f(sc[u][h] - m[h]);
                l[h] += w;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[h][e] = fmaf(w, vf[e], acc[h][e]);
            }
        }
    };

    // ---- the pipeline: iteration i issues entries(i+2), pages(i+1), rows(i) and
    // folds rows(i-1). Register sets alternate between even and odd iterations.
    if (nb > 0) {
        Entries E0, E1;
        Pages P0, P1;
        Rows R0, R1;
        load_entries(0, E0);
        load_entries(1, E1);
        load_pages(0, E0, P0);
        // iterations 0 and 1 are peeled so that the loop is entered with the same
        // loads in flight as at its back edge
        load_entries(2, E0);
        load_pages(1, E1, P1);
        load_rows(P0, R0);
        load_entries(3, E1);
        load_pages(2, E0, P0);
        load_rows(P1, R1);
        consume(R0);
        for (int i = 2; i <= nb; i += 2) {
            load_entries(i + 2, E0);
            load_pages(i + 1, E1, P1);
            load_rows(P0, R0);
            consume(R1);
            if (i + 1 > nb)
                break;
            load_entries(i + 3, E1);
            load_pages(i + 2, E0, P0);
            load_rows(P1, R1);
            consume(R0);
        }
    }

    // merge the key teams of this wavefront
#pragma unroll
    for (int off = TL; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m2 = __shfl_xor(m[h], off);
            const float l2 = __shfl_xor(l[h], off);
            const float mn = fmaxf(m[h], m2);
            const float c1 = __builtin_amdgcn_exp2f(m[h] - mn);
            const float c2 = __builtin_amdgcn_exp2f(m2 - mn);
            l[h] = c1 * l[h] + c2 * l2;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[h][e] = c1 * acc[h][e] + c2 * __shfl_xor(acc[h][e], off);
            m[h] = mn;
        }
    }

    // merge the wavefronts through LDS
    float *s_ml = smem;                          // [NW][G][2]
    float *s_acc = smem + kMaxWaves * G * 2;     // [NW][G][D]
    if (lane < TL) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (lane == 0) {
                s_ml[(wave * G + h) * 2] = m[h];
                s_ml[(wave * G + h) * 2 + 1] = l[h];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                s_acc[(wave * G + h) * D + lane * EPL + e] = acc[h][e];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += nthreads) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = kNoKey;
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, s_ml[(w * G + h) * 2]);
        float L = 0.f, A = 0.f;
        for (int w = 0; w < NW; ++w) {
            const float c = __builtin_amdgcn_exp2f(s_ml[(w * G + h) * 2] - M);
            L += c * s_ml[(w * G + h) * 2 + 1];
            A += c * s_acc[(w * G + h) * D + d];
        }
        const int64_t rh = r * p.num_q_heads + (int64_t)g * G + h;
        if (S == 1) {
            store_out(p.out, p.out_dtype, rh * D + d, A * final_factor(p, (int64_t)g * G + h, M, L));
        } else {
            const int64_t srh = (int64_t)s * p.total_q * p.num_q_heads + rh;
            p.ws_acc[srh * D + d] = A;
            if (d == 0) {
                p.ws_ml[srh * 2] = M;
                p.ws_ml[srh * 2 + 1] = L;
            }
        }
    }
}

template <int DT, int D, int G, int U, int LIST>
int launch_valu(const GatherParams &p, void *stream)
{
    const int64_t grid = p.total_q * (int64_t)p.num_kv_heads * p.num_splits;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gather_valu_kernel<DT, D, G, U, LIST>), dim3((unsigned)grid), dim3(64 * p.waves),
                       0, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

template <int DT, int D, int G, int LIST>
int launch_valu_u(const GatherParams &p, void *stream)
{
    if (p.unroll >= 4)
        return launch_valu<DT, D, G, 4, LIST>(p, stream);
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

template <int LIST>
int launch_valu_t(const GatherParams &p, void *stream)
{
    switch (p.dtype) {
    case QSA_F32: return launch_valu_d<QSA_F32, LIST>(p, stream);
    case QSA_BF16: return launch_valu_d<QSA_BF16, LIST>(p, stream);
    case QSA_FP8_E4M3: return launch_valu_d<QSA_FP8_E4M3, LIST>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace

bool valu_supported(int32_t dtype, int32_t group, int32_t head_dim)
{
    return (dtype == QSA_F32 || dtype == QSA_BF16 || dtype == QSA_FP8_E4M3) &&
           (group == 1 || group == 2 || group == 4) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

int launch_gather_valu(const GatherParams &p, void *stream)
{
    switch (p.list_kind) {
    case KEYS_TOKEN_INDICES: return launch_valu_t<KEYS_TOKEN_INDICES>(p, stream);
    case KEYS_BLOCKS: return launch_valu_t<KEYS_BLOCKS>(p, stream);
    case KEYS_LATENT: return launch_valu_t<KEYS_LATENT>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace qsa
