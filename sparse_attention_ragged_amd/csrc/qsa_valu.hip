// Gather-attention kernel on wavefront dot products (groups of 1, 2 or 4 query
// heads per kv head).
//
// One workgroup owns one (query row, kv head, split) and walks that split of the
// row's key list ("QSASparseAttentionRaggedPaged": token_indices up to counts;
// "Struct_msa_attention_ragged_paged": the positions of the listed blocks up to the
// row's position; "latent_sparse_attention_ragged_paged": window positions, then
// listed compressed entries).
//
//  1. Address generation: the workgroup turns up to 1024 list entries at a time into
//     byte addresses of their K rows (index -> page table -> 64-bit address) and
//     stages them in LDS, so the gather loop never waits on that dependent chain.
//  2. Gather + online softmax: a "key team" of TL = head_dim * elem_bytes / 16 lanes
//     owns one key at a time; every lane issues one 16-byte load for K and one for V.
//     A team keeps U keys in flight (the pages' `unroll`), reduces each head's partial
//     dot product across its lanes with DPP, and folds the U keys into a running
//     (max, sum, acc) state per query head, in fp32 and in the log2 domain.
//  3. Merge: teams of a wavefront merge their states with lane shuffles, wavefronts
//     through LDS; the result is either the normalised output row (one split) or an
//     (m, l, acc) partial for the split-K combine kernel.
#include "qsa_device.hpp"

namespace qsa {

namespace {

constexpr int kStageKeys = 1024;
constexpr int kMaxWaves = 8;

template <int DT, int D, int G, int U>
__global__ void __launch_bounds__(64 * kMaxWaves) gather_valu_kernel(GatherParams p)
{
    constexpr int EB = Elem<DT>::bytes;
    constexpr int EPL = 16 / EB;   // elements of a row held by one lane
    constexpr int TL = D / EPL;    // lanes per key team
    static_assert(TL >= 1 && TL <= 64 && 64 % TL == 0, "unsupported head_dim for this dtype");
    constexpr int kMergeBytes = kMaxWaves * G * (D + 2) * 4;
    constexpr int kSmem = kStageKeys * 8 > kMergeBytes ? kStageKeys * 8 : kMergeBytes;
    __shared__ __attribute__((aligned(16))) char smem[kSmem];
    const char **s_addr = reinterpret_cast<const char **>(smem);

    const int S = p.num_splits;
    const int Hkv = p.num_kv_heads;
    int64_t bid = blockIdx.x;
    const int g = (int)(bid % Hkv);
    bid /= Hkv;
    const int s = (int)(bid % S);
    const int64_t r = bid / S;
    const int b = find_seq(p.row_off, p.batch, (uint32_t)r);
    const int64_t pos = (int64_t)p.cache_lengths[b] + (r - (int64_t)p.row_off[b]);
    const int64_t n = key_list_length(p, r);
    const int64_t j0 = (int64_t)s * p.split_keys;
    const int64_t j1 = n < j0 + p.split_keys ? n : j0 + p.split_keys;

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int team = tid / TL;
    const int ln = tid % TL;
    const int NT = nthreads / TL;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int NW = nthreads >> 6;
    const int64_t vdelta = p.list_kind == KEYS_LATENT ? 0 : p.kv.plane_stride * EB;

    // this lane's slice of the G query rows of kv head g
    const int64_t qrow = (r * p.num_q_heads + (int64_t)g * G) * D;
    u32x4 qraw[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        qraw[h] = ldg16(static_cast<const char *>(p.q) + (qrow + (int64_t)h * D + ln * EPL) * EB);
    float qf[(DT == QSA_BF16) ? 1 : G][(DT == QSA_BF16) ? 1 : EPL];
    if constexpr (DT == QSA_F32) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qf[h][i] = __uint_as_float(qraw[h][i]);
    } else if constexpr (DT == QSA_FP8_E4M3) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                e4m3x4_to_f32(qraw[h][i], &qf[h][4 * i]);
    }

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = kNegInf;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            acc[h][e] = 0.f;
    }

    for (int64_t c0 = j0; c0 < j1; c0 += kStageKeys) {
        const int clen = (int)(j1 - c0 < kStageKeys ? j1 - c0 : kStageKeys);
        __syncthreads();
        for (int i = tid; i < clen; i += nthreads)
            s_addr[i] = key_address<EB>(p, b, r, pos, g, c0 + i);
        __syncthreads();

        for (int base = 0; base < clen; base += NT * U) {
            u32x4 kr[U], vr[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int j = base + u * NT + team;
                const char *a = j < clen ? s_addr[j] : nullptr;
                ok[u] = a != nullptr;
                if (ok[u]) {
                    kr[u] = ldg16(a + ln * 16);
                    vr[u] = ldg16(a + vdelta + ln * 16);
                } else {
                    kr[u] = u32x4{0, 0, 0, 0};
                    vr[u] = u32x4{0, 0, 0, 0};
                }
            }
            float sc[U][G];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float kf[(DT == QSA_BF16) ? 1 : EPL];
                if constexpr (DT == QSA_F32) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        kf[i] = __uint_as_float(kr[u][i]);
                } else if constexpr (DT == QSA_FP8_E4M3) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        e4m3x4_to_f32(kr[u][i], &kf[4 * i]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float d = 0.f;
                    if constexpr (DT == QSA_BF16) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qraw[h][i]),
                                                                as_bf16x2(kr[u][i]), d, false);
                    } else {
#pragma unroll
                        for (int i = 0; i < EPL; ++i)
                            d = fmaf(qf[h][i], kf[i], d);
                    }
                    d = team_sum<TL>(d) * p.scale_log2;
                    sc[u][h] = ok[u] ? d : kNegInf;
                }
            }
            float vf[U][EPL];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (DT == QSA_F32) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vf[u][i] = __uint_as_float(vr[u][i]);
                } else if constexpr (DT == QSA_BF16) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        vf[u][2 * i] = bf16_lo(vr[u][i]);
                        vf[u][2 * i + 1] = bf16_hi(vr[u][i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        e4m3x4_to_f32(vr[u][i], &vf[u][4 * i]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float mx = m[h];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    mx = fmaxf(mx, sc[u][h]);
                const float ref = mx == kNegInf ? 0.f : mx;
                const float alpha = __builtin_amdgcn_exp2f(m[h] - ref);
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e)
                    acc[h][e] *= alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float w = __builtin_amdgcn_exp2f(sc[u][h] - ref);
                    l[h] += w;
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        acc[h][e] = fmaf(w, vf[u][e], acc[h][e]);
                }
                m[h] = mx;
            }
        }
    }

    // merge the key teams of this wavefront
#pragma unroll
    for (int off = TL; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m2 = __shfl_xor(m[h], off);
            const float l2 = __shfl_xor(l[h], off);
            float c1, c2, mn;
            merge_scale(m[h], m2, c1, c2, mn);
            l[h] = c1 * l[h] + c2 * l2;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[h][e] = c1 * acc[h][e] + c2 * __shfl_xor(acc[h][e], off);
            m[h] = mn;
        }
    }

    // merge the wavefronts through LDS
    float *s_ml = reinterpret_cast<float *>(smem);          // [NW][G][2]
    float *s_acc = s_ml + kMaxWaves * G * 2;                 // [NW][G][D]
    __syncthreads();
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
        float M = kNegInf;
        for (int w = 0; w < NW; ++w)
            M = fmaxf(M, s_ml[(w * G + h) * 2]);
        const float ref = M == kNegInf ? 0.f : M;
        float L = 0.f, A = 0.f;
        for (int w = 0; w < NW; ++w) {
            const float c = __builtin_amdgcn_exp2f(s_ml[(w * G + h) * 2] - ref);
            L += c * s_ml[(w * G + h) * 2 + 1];
            A += c * s_acc[(w * G + h) * D + d];
        }
        const int64_t rh = r * p.num_q_heads + (int64_t)g * G + h;
        if (S == 1) {
            store_out(p.out, p.out_dtype, rh * D + d, L > 0.f ? A / L : 0.f);
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

template <int DT, int D, int G, int U>
int launch_valu(const GatherParams &p, void *stream)
{
    const int64_t grid = p.total_q * (int64_t)p.num_kv_heads * p.num_splits;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gather_valu_kernel<DT, D, G, U>), dim3((unsigned)grid), dim3(64 * p.waves),
                       0, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

template <int DT, int D, int G>
int launch_valu_u(const GatherParams &p, void *stream)
{
    // the decode-shaped bf16 instantiation carries every unroll; the rest use 4
    if constexpr (DT == QSA_BF16 && D == 128 && G == 4) {
        switch (p.unroll) {
        case 2: return launch_valu<DT, D, G, 2>(p, stream);
        case 8: return launch_valu<DT, D, G, 8>(p, stream);
        default: return launch_valu<DT, D, G, 4>(p, stream);
        }
    } else {
        return launch_valu<DT, D, G, 4>(p, stream);
    }
}

template <int DT, int D>
int launch_valu_g(const GatherParams &p, void *stream)
{
    switch (p.group) {
    case 1: return launch_valu_u<DT, D, 1>(p, stream);
    case 2: return launch_valu_u<DT, D, 2>(p, stream);
    case 4: return launch_valu_u<DT, D, 4>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

template <int DT>
int launch_valu_d(const GatherParams &p, void *stream)
{
    switch (p.head_dim) {
    case 64: return launch_valu_g<DT, 64>(p, stream);
    case 128: return launch_valu_g<DT, 128>(p, stream);
    case 256: return launch_valu_g<DT, 256>(p, stream);
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
    switch (p.dtype) {
    case QSA_F32: return launch_valu_d<QSA_F32>(p, stream);
    case QSA_BF16: return launch_valu_d<QSA_BF16>(p, stream);
    case QSA_FP8_E4M3: return launch_valu_d<QSA_FP8_E4M3>(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace qsa
