// Split-K combine ("Struct_msa_attention_ragged_paged" design notes: decode runs
// over partitioned KV bands and then merges them in a reduction kernel).
//
// Each split s left, for every (row, q head), a log2-domain reference m_s (at least the
// largest score it saw minus a small slack, or a large negative value if it saw no
// key), the sum
// l_s = sum_j 2^(t_j - m_s) and acc_s = sum_j 2^(t_j - m_s) V_j. The exact result is
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// and a (row, head) that saw no key anywhere (l = 0 everywhere) is written as zeros.
// A per-head sink logit (latent attention) joins the denominator here, once.
#include "qsa_device.hpp"

namespace qsa {

namespace {

__global__ void __launch_bounds__(256) splitk_combine_kernel(GatherParams p)
{
    const int D = p.head_dim;
    const int tpr = D / 4;                     // threads per (row, head), 4 values each
    const int per_block = 256 / tpr;
    // partials exist for the rows from split_row0 on (all rows unless a tail plan ran
    // the earlier ones unsplit); they are indexed relative to that row
    const int64_t RH = (p.total_q - p.split_row0) * p.num_q_heads;
    const int64_t rel = (int64_t)blockIdx.x * per_block + threadIdx.x / tpr;
    const int64_t rh = p.split_row0 * p.num_q_heads + rel;
    const int d0 = (threadIdx.x % tpr) * 4;
    if (rel >= RH || threadIdx.x / tpr >= per_block)
        return;
    const int S = p.num_splits;
    float M = kNoKey;
    // unrolled so that several partials' loads are in flight at once
#pragma unroll 8
    for (int s = 0; s < S; ++s)
        M = fmaxf(M, p.ws_ml[((int64_t)s * RH + rel) * 2]);
    float L = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
        const int64_t srh = (int64_t)s * RH + rel;
        const float c = __builtin_amdgcn_exp2f(p.ws_ml[srh * 2] - M);
        L += c * p.ws_ml[srh * 2 + 1];
        const float4 v = *reinterpret_cast<const float4 *>(p.ws_acc + srh * D + d0);
        a0 += c * v.x;
        a1 += c * v.y;
        a2 += c * v.z;
        a3 += c * v.w;
    }
    const float f = final_factor(p, rh % p.num_q_heads, M, L);
    const int64_t o = rh * D + d0;
    store_out(p.out, p.out_dtype, o + 0, a0 * f);
    store_out(p.out, p.out_dtype, o + 1, a1 * f);
    store_out(p.out, p.out_dtype, o + 2, a2 * f);
    store_out(p.out, p.out_dtype, o + 3, a3 * f);
}

}  // namespace

int launch_splitk_combine(const GatherParams &p, void *stream)
{
    const int64_t RH = (p.total_q - p.split_row0) * p.num_q_heads;
    if (RH == 0)
        return 0;
    if (p.head_dim % 4 != 0 || p.head_dim / 4 > 256)
        return (int)hipErrorInvalidValue;
    const int per_block = 256 / (p.head_dim / 4);
    const int64_t grid = (RH + per_block - 1) / per_block;
    if (grid > 0x7fffffff)
        return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(splitk_combine_kernel, dim3((unsigned)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), p);
    return (int)hipGetLastError();
}

int record_event(void *event, void *stream)
{
    return (int)hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream));
}

const char *hip_error_text(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace qsa
