// Per-team core of the wavefront gather kernels (groups of 1, 2 or 4 query heads per
// kv head): the register layout of a key's K/V rows over a team of lanes, the scoring
// of a batch of U keys per team against the q rows, the online-softmax fold and the
// merge of teams, run by the wavefront gather kernel (one workgroup per (row, kv
// head, split)).
//
//  * Teams: a team of TL lanes owns one (key, kv head) at a time; each lane holds CPL
//    16-byte chunks of the K row and of the V row (chunk c of lane l is chunk c*TL + l
//    of the row, so one load instruction reads TL consecutive chunks). Two chunks per
//    lane (bf16, fp32) halve the per-key address arithmetic and shorten the team
//    reduction.
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
#pragma once

#include <type_traits>

#include "qsa_device.hpp"

namespace qsa {

constexpr float kValuRescaleSlack = 8.0f;   // log2 units: weights stay <= 2^8

template <int DT, int D, int G, int U>
struct ValuCore {
    static constexpr int EB = Elem<DT>::bytes;
    static constexpr int EPC = 16 / EB;                    // elements per chunk
    // 16-byte chunks per lane: two where a lane then holds at most 16 elements (bf16,
    // fp32); e4m3 keeps one (its q is widened to fp32 in registers)
    static constexpr int CPL = valu_chunks_per_lane(EB, D);
    static constexpr int TL = valu_team_lanes(EB, D);      // lanes per team
    static constexpr int TPW = 64 / TL;                    // teams per wavefront
    static constexpr int EPL = EPC * CPL;                  // elements per lane
    static constexpr int QF = DT == QSA_BF16 ? 1 : EPL;    // widened q elements per lane
    static constexpr bool kPaired = DT == QSA_BF16 && U % 2 == 0;
    static_assert(TL >= 4 && TL <= 64 && 64 % TL == 0, "unsupported head_dim for this dtype");

    // element offset of chunk c of lane `ln` (lane within its team) within a row
    __device__ __forceinline__ static int chunk_elem(int c, int ln) { return (c * TL + ln) * EPC; }

    // this lane's chunks of the G q rows (raw words; widened to fp32 unless bf16)
    struct Q {
        u32x4 raw[G][CPL];
        float f[G][QF];
    };
    // this lane's chunks of the K and V rows of U keys, and which keys are present
    struct Rows {
        u32x4 k[U][CPL], v[U][CPL];
        bool ok[U];
    };

    float m[G], l[G], acc[G][EPL];

    __device__ __forceinline__ void reset()
    {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = kNoKey;
            l[h] = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                acc[h][e] = 0.f;
        }
    }

    __device__ __forceinline__ static void widen_q(Q &q)
    {
        if constexpr (DT != QSA_BF16) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int c = 0; c < CPL; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if constexpr (DT == QSA_F32)
                            q.f[h][c * EPC + i] = __uint_as_float(q.raw[h][c][i]);
                        else
                            e4m3x4_to_f32(q.raw[h][c][i], &q.f[h][c * EPC + 4 * i]);
                    }
        }
    }

    // fold the U keys of R into the running state
    __device__ __forceinline__ void consume(const Rows &R, const Q &q, float scale_log2)
    {
        float sc[U][G];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[QF];
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
                            d = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.raw[h][c][i]), as_bf16x2(R.k[u][c][i]),
                                                                d, false);
                } else {
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        d = fmaf(q.f[h][e], kf[e], d);
                }
                d = team_sum<TL>(d) * scale_log2;
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
            need |= mx[h] > m[h] + kValuRescaleSlack;
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
    }

    // merge with the team OFF lanes away (butterfly step)
    template <int OFF>
    __device__ __forceinline__ void merge_pair()
    {
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
    }

    // merge the teams of a wavefront whose lanes are `span` or more apart (teams of the
    // same kv head sit span lanes apart): afterwards every such team holds the
    // wavefront's state for its head
    __device__ __forceinline__ void merge_teams(int span)
    {
        if constexpr (TL <= 4) if (4 >= span) merge_pair<4>();
        if constexpr (TL <= 8) if (8 >= span) merge_pair<8>();
        if constexpr (TL <= 16) if (16 >= span) merge_pair<16>();
        if constexpr (TL <= 32) if (32 >= span) merge_pair<32>();
    }
};

}  // namespace qsa
