// Split-K combine kernel ("Struct_msa_attention_ragged_paged" design notes: decode runs
// over partitioned KV bands and then merges them in a reduction kernel), for plans
// whose splits do not merge themselves (see merge_splits4). One thread per four
// outputs of a (row, head).
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
    if (rel >= RH || threadIdx.x / tpr >= per_block)
        return;
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
