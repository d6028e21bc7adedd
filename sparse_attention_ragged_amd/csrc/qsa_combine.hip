// Split-K combine kernel ("Struct_msa_attention_ragged_paged" design notes: decode runs
// over partitioned KV bands and then merges them in a reduction kernel), for plans
// whose splits do not merge themselves. One thread per four outputs of a (row, head).
#include "qsa_device.hpp"

namespace qsa {

namespace {

// The merge for at most SMAX splits: every split's (m, l) pair and four accumulator
// values are loaded at once (a split index past num_splits re-reads the last split and
// gets weight 0), so the loads form one round instead of the (m) round and the (l, acc)
// round of the general merge. The same sums in the same order.
template <int SMAX>
__device__ __forceinline__ void merge_splits4_fixed(const GatherParams &p, int64_t rh, int64_t rel, int d0)
{
    const int S = p.num_splits;
    const int D = p.head_dim;
    const int64_t RH = (p.total_q - p.split_row0) * p.num_q_heads;
    float mv[SMAX], lv[SMAX];
    f32x4_t av[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
        const int64_t srh = (int64_t)(s < S ? s : S - 1) * RH + rel;
        typedef float f32x2v __attribute__((ext_vector_type(2)));
        const f32x2v ml = *reinterpret_cast<const f32x2v *>(p.ws_ml + srh * 2);
        mv[s] = ml[0];
        lv[s] = ml[1];
        av[s] = *reinterpret_cast<const f32x4_t *>(p.ws_acc + srh * D + d0);
    }
    float M = kNoKey;
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
        M = fmaxf(M, s < S ? mv[s] : kNoKey);
    float L = 0.f;
    f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
        const float c = s < S ? __builtin_amdgcn_exp2f(mv[s] - M) : 0.f;
        L += c * lv[s];
        a += c * av[s];
    }
    store_out4(p.out, p.out_dtype, rh * D + d0, a * final_factor(p, rh % p.num_q_heads, M, L));
}

template <int SMAX>
__global__ void __launch_bounds__(256) splitk_combine_kernel(GatherParams p)
{
    const int D = p.head_dim;
    const int tpr = D / 4;                     // threads per (row, head), 4 values each
    const int per_block = 256 / tpr;
    // partials exist for the rows from split_row0 on (all rows unless a tail plan ran
    // the earlier ones unsplit); they are indexed relative to that row
    const int64_t RH = (p.total_q - p.split_row0) * p.num_q_heads;
    const int64_t rel = (int64_t)blockIdx.x * per_block + threadIdx.x / tpr;
    if (rel >= RH || threadIdx.x / tpr >= per_block)
        return;
    if constexpr (SMAX > 0)
        merge_splits4_fixed<SMAX>(p, p.split_row0 * p.num_q_heads + rel, rel, (threadIdx.x % tpr) * 4);
    else
        merge_splits4(p, p.split_row0 * p.num_q_heads + rel, rel, (threadIdx.x % tpr) * 4);
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
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.num_splits <= 8)
        hipLaunchKernelGGL(splitk_combine_kernel<8>, dim3((unsigned)grid), dim3(256), 0, st, p);
    else if (p.num_splits <= 16)
        hipLaunchKernelGGL(splitk_combine_kernel<16>, dim3((unsigned)grid), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL(splitk_combine_kernel<0>, dim3((unsigned)grid), dim3(256), 0, st, p);
    return (int)hipGetLastError();
}

int record_event(void *event, void *stream)
{
    return (int)hipEventRecord(static_cast<hipEvent_t>(event), static_cast<hipStream_t>(stream));
}

const char *hip_error_text(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

}  // namespace qsa
