// Gather-attention kernel on wavefront dot products (groups of 1, 2 or 4 query
// heads per kv head).
//
// One workgroup owns one (query row, kv head, split) and walks that split of the
// row's key list ("QSASparseAttentionRaggedPaged": token_indices up to counts;
// "Struct_msa_attention_ragged_paged": the positions of the listed blocks up to the
// row's position; "latent_sparse_attention_ragged_paged": window positions, then
// listed compressed entries).
//
//  * Teams: a team of TL lanes owns one (key, kv head) at a time; each lane holds CPL
//    16-byte chunks of the K row and of the V row (chunk c of lane l is chunk c*TL + l
//    of the row, so one load instruction reads TL consecutive chunks). Two chunks per
//    lane (bf16, fp32) halve the per-key address arithmetic and shorten the team
//    reduction.
//  * Head blocks: when all kv heads read the same keys (token-index and latent
//    lists), a workgroup covers a block of HB kv heads and the teams of a wavefront
//    are HB heads x (64/TL/HB) key slots. At HB = 8 (bf16, head_dim 128, 8 kv heads) a
//    wavefront reads a key's whole K block and V block (all heads, contiguous in the
//    page) with one request each, and the key's address is computed once per
//    wavefront. Key slots take keys j0 + b*NK*U + u*NK + slot (batch b, u < U, NK slots
//    per workgroup).
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
//  * P.V for bf16: the weights of two keys are rounded to bf16 and paired, the two
//    keys' V elements are paired with byte permutes, and one packed bf16 dot
//    instruction adds both products in fp32; the running sum adds the same rounded
//    weights, so numerator and denominator use identical weights. fp32 and e4m3 use
//    fp32 FMAs on the widened values.
//  * Merge: teams of a wavefront merge with lane shuffles, wavefronts through LDS;
//    the result is the normalised output row (one split) or an (m, l, acc) partial
//    for the split-K combine kernel.
#include <atomic>
#include <type_traits>

#include "qsa_device.hpp"

namespace qsa {

namespace {

constexpr int kMaxWaves = 8;
constexpr float kRescaleSlack = 8.0f;   // log2 units: weights stay <= 2^8

template <int DT, int D, int G, int U, int LIST>
__global__ void __launch_bounds__(64 * kMaxWaves) gather_valu_kernel(GatherParams p)
{
    constexpr int EB = Elem<DT>::bytes;
    constexpr int EPC = 16 / EB;                 // elements per chunk
    // 16-byte chunks per lane: two where a lane then holds at most 16 elements (bf16,
    // fp32); e4m3 keeps one (its q is widened to fp32 in registers)
    constexpr int CPL = valu_chunks_per_lane(EB, D);
    constexpr int TL = valu_team_lanes(EB, D);   // lanes per team
    constexpr int TPW = 64 / TL;                 // teams per wavefront
    constexpr int EPL = EPC * CPL;               // elements per lane
    constexpr bool kPaired = DT == QSA_BF16 && U % 2 == 0;
    static_assert(TL >= 1 && TL <= 64 && 64 % TL == 0, "unsupported head_dim for this dtype");
    extern __shared__ __attribute__((aligned(16))) float smem[];   // [NW][HB*G][2], then [NW][HB*G][D]

    const int S = p.num_splits;
    const int HB = p.head_block;                 // kv heads of this workgroup, one team each
    int64_t bid = blockIdx.x;
    const int nhb = p.num_kv_heads / HB;
    const int gb = (int)(bid % nhb);
    bid /= nhb;
    const int s = (int)(bid % S);
    const int64_t r = bid / S;

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

    // element offset of chunk c of this lane within a row
    auto chunk_elem = [&](int c) { return (c * TL + ln) * EPC; };

    // prologue: list length, sequence and the q rows go out together
    const int64_t n = key_list_length(p, r);
    const char *qbase = static_cast<const char *>(p.q) + ((r * p.num_q_heads + (int64_t)g * G) * D) * EB;
    u32x4 qraw[G][CPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            qraw[h][c] = ldg16(qbase + ((int64_t)h * D + chunk_elem(c)) * EB);
    const int b = find_seq_wave(p.row_off, p.batch, (uint32_t)r);
    int64_t pos = 0;
    if constexpr (LIST != KEYS_TOKEN_INDICES)
        pos = (int64_t)p.cache_lengths[b] + (r - (int64_t)p.row_off[b]);
    const int64_t j0 = (int64_t)s * p.split_keys;
    const int64_t j1 = n < j0 + p.split_keys ? n : j0 + p.split_keys;
    const int64_t per_batch = (int64_t)NK * U;
    const int nb = j1 > j0 ? (int)((j1 - j0 + per_batch - 1) / per_batch) : 0;
    const int64_t vdelta = LIST == KEYS_LATENT ? 0 : (int64_t)p.kv.plane_stride_b;
    const char *dummy = qbase;                   // a readable row for absent keys

    float qf[G][DT == QSA_BF16 ? 1 : EPL];
    if constexpr (DT != QSA_BF16) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (DT == QSA_F32)
                        qf[h][c * EPC + i] = __uint_as_float(qraw[h][c][i]);
                    else
                        e4m3x4_to_f32(qraw[h][c][i], &qf[h][c * EPC + 4 * i]);
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
    struct Rows { u32x4 k[U][CPL], v[U][CPL]; bool ok[U]; };

    auto key_index = [&](int batch, int u) -> int64_t {
        return j0 + batch * per_batch + u * NK + wave * KPW + ks;
    };
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
            const char *base = ok ? a : dummy;
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                R.k[u][c] = ldg16(base + (int64_t)chunk_elem(c) * EB);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                R.v[u][c] = ldg16((ok ? a + vdelta : dummy) + (int64_t)chunk_elem(c) * EB);
        }
    };
    auto consume = [&](const Rows &R) {
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[DT == QSA_BF16 ? 1 : EPL];
            if constexpr (DT != QSA_BF16) {
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (DT == QSA_F32)
                            kf[c * EPC + i] = __uint_as_float(R.k[u][c][i]);
                        else
                            e4m3x4_to_f32(R.k[u][c][i], &kf[c * EPC + 4 * i]);
                    }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
                if constexpr (DT == QSA_BF16) {
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qraw[h][c][i]), as_bf16x2(R.k[u][c][i]),
                                                                d, false);
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
        if constexpr (kPaired) {
#pragma unroll
            for (int u = 0; u < U; u += 2) {
                // (key u, key u+1) pairs of each V element
                uint32_t vlo[CPL][4], vhi[CPL][4];
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        vlo[c][i] = __builtin_amdgcn_perm(R.v[u + 1][c][i], R.v[u][c][i], 0x05040100u);
                        vhi[c][i] = __builtin_amdgcn_perm(R.v[u + 1][c][i], R.v[u][c][i], 0x07060302u);
                    }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint32_t wp = pack_bf16x2(__builtin_amdgcn_exp2f(sc[u][h] - m[h]),
                                                    __builtin_amdgcn_exp2f(sc[u + 1][h] - m[h]));
                    l[h] += bf16_lo(wp) + bf16_hi(wp);
                    const bf16x2_t w2 = as_bf16x2(wp);
#pragma unroll
                    for (int c = 0; c < CPL; ++c)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float &a0 = acc[h][c * EPC + 2 * i];
                            float &a1 = acc[h][c * EPC + 2 * i + 1];
                            a0 = __builtin_amdgcn_fdot2_f32_bf16(w2, as_bf16x2(vlo[c][i]), a0, false);
                            a1 = __builtin_amdgcn_fdot2_f32_bf16(w2, as_bf16x2(vhi[c][i]), a1, false);
                        }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float vf[EPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (DT == QSA_F32) {
                            vf[c * EPC + i] = __uint_as_float(R.v[u][c][i]);
                        } else if constexpr (DT == QSA_BF16) {
                            vf[c * EPC + 2 * i] = bf16_lo(R.v[u][c][i]);
                            vf[c * EPC + 2 * i + 1] = bf16_hi(R.v[u][c][i]);
                        } else {
                            e4m3x4_to_f32(R.v[u][c][i], &vf[c * EPC + 4 * i]);
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

    // merge the key slots of this wavefront (butterfly over teams of the same kv head:
    // afterwards every such team holds the wavefront's state for its head)
    auto merge_teams = [&](auto off_tag) {
        constexpr int OFF = decltype(off_tag)::value;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float ma, mb, la, lb;
            xor_pair<OFF>(m[h], ma, mb);
            xor_pair<OFF>(l[h], la, lb);
            const float mn = fmaxf(ma, mb);
            const float ca = __builtin_amdgcn_exp2f(ma - mn);
            const float cb = __builtin_amdgcn_exp2f(mb - mn);
            l[h] = ca * la + cb * lb;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                float aa, ab;
                xor_pair<OFF>(acc[h][e], aa, ab);
                acc[h][e] = ca * aa + cb * ab;
            }
            m[h] = mn;
        }
    };
    // teams of the same kv head sit TL*HB lanes apart
    if constexpr (TL <= 4) if (4 >= TL * HB) merge_teams(std::integral_constant<int, 4>());
    if constexpr (TL <= 8) if (8 >= TL * HB) merge_teams(std::integral_constant<int, 8>());
    if constexpr (TL <= 16) if (16 >= TL * HB) merge_teams(std::integral_constant<int, 16>());
    if constexpr (TL <= 32) if (32 >= TL * HB) merge_teams(std::integral_constant<int, 32>());
    static_assert(TL >= 4, "team merge starts at 4-lane teams");

    // merge the wavefronts through LDS: the key-slot-0 team of each kv head writes it
    const int HG = HB * G;                       // q heads of the workgroup
    float *s_ml = smem;                          // [NW][HG][2]
    float *s_acc = smem + ((NW * HG * 2 + 3) & ~3);   // [NW][HG][D], 16-byte aligned
    if (ks == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const int hq = hh * G + h;
            if (ln == 0) {
                s_ml[(wave * HG + hq) * 2] = m[h];
                s_ml[(wave * HG + hq) * 2 + 1] = l[h];
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c)
#pragma unroll
                for (int e = 0; e < EPC; e += 4)
                    *reinterpret_cast<float4 *>(&s_acc[(wave * HG + hq) * D + chunk_elem(c) + e]) =
                        make_float4(acc[h][c * EPC + e], acc[h][c * EPC + e + 1], acc[h][c * EPC + e + 2],
                                    acc[h][c * EPC + e + 3]);
        }
    }
    __syncthreads();
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

template <int DT, int D, int G, int U, int LIST>
int launch_valu(const GatherParams &p, void *stream)
{
    const int64_t grid = p.total_q * (int64_t)(p.num_kv_heads / p.head_block) * p.num_splits;
    if (grid <= 0)
        return 0;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    // LDS of the cross-wavefront merge: (reference, sum) and D partial outputs per q head
    const size_t hg = (size_t)p.waves * p.head_block * G;
    const size_t lds = (((2 * hg + 3) & ~(size_t)3) + hg * D) * sizeof(float);
    // allow more than the default dynamic LDS, once per device
    static std::atomic<uint64_t> raised{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        dev = 63;
    if (!(raised.load() >> dev & 1u)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gather_valu_kernel<DT, D, G, U, LIST>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess)
            return (int)e;
        raised.fetch_or(uint64_t(1) << dev);
    }
    hipLaunchKernelGGL((gather_valu_kernel<DT, D, G, U, LIST>), dim3((unsigned)grid), dim3(64 * p.waves),
                       lds, static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
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
