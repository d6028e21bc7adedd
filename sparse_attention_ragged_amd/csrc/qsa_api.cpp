// extern "C" entry points declared in include/qsa.h: check arguments on the host,
// plan the launch, fill the parameter block and hand it to the kernel launchers.
// No HIP headers here; all device work goes through the launchers.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "qsa_host.hpp"
#include "qsa_select_host.hpp"
#include "qsa_flash_host.hpp"

namespace qsa {
const char *last_error_text();
}

using namespace qsa;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

thread_local void *t_ev_start = nullptr;
thread_local void *t_ev_stop = nullptr;

void fill_common(GatherParams &p, void *out, int32_t out_dtype, const qsa_ragged_q *q,
                 int64_t num_kv_heads, uint32_t layer, float scale, const Plan &plan, void *ws)
{
    std::memset(&p, 0, sizeof p);
    p.out = out;
    p.out_dtype = out_dtype;
    p.dtype = q->dtype;
    p.q = q->q;
    p.total_q = q->total_q;
    p.num_q_heads = (int32_t)q->num_q_heads;
    p.num_kv_heads = (int32_t)num_kv_heads;
    p.head_dim = (int32_t)q->head_dim;
    p.group = (int32_t)(q->num_q_heads / num_kv_heads);
    p.batch = (int32_t)q->batch;
    p.layer = (int32_t)layer;
    p.row_off = q->input_row_offsets;
    p.scale_log2 = scale * 1.44269504088896340736f;
    p.num_splits = plan.num_splits;
    p.waves = plan.waves;
    p.unroll = plan.unroll;
    p.split_keys = plan.split_keys;
    p.split_row0 = plan.split_row0;
    p.head_block = plan.head_block;
    p.stream_rows = plan.stream_rows;
    if (plan.num_splits > 1) {
        p.ws_acc = static_cast<float *>(ws);
        p.ws_ml = reinterpret_cast<float *>(static_cast<char *>(ws) + plan.ws_ml_offset);
    }
}

qsa_status run(const GatherParams &p, const Plan &plan, void *stream)
{
    if (p.total_q == 0)
        return QSA_OK;
    int err = 0;
    if (t_ev_start && t_ev_stop)
        err = record_event(t_ev_start, stream);
    if (!err)
        err = plan.path == PATH_MFMA_WIDE ? launch_gather_mfma_wide(p, stream)
              : plan.path == PATH_MFMA    ? launch_gather_mfma(p, stream)
                                          : launch_gather_valu(p, stream);
    if (!err && t_ev_start && t_ev_stop)
        err = record_event(t_ev_stop, stream);
    if (!err && plan.num_splits > 1)
        err = launch_splitk_combine(p, stream);
    if (err)
        return fail(QSA_ERR_HIP, "HIP launch failed: %s", hip_error_text(err));
    return QSA_OK;
}

qsa_status check_out(void *out, int32_t out_dtype, const qsa_ragged_q *q)
{
    if (q->total_q > 0 && !out)
        return fail(QSA_ERR_NULL, "out is NULL");
    if (out_dtype != QSA_F32 && out_dtype != QSA_BF16)
        return fail(QSA_ERR_DTYPE, "out_dtype must be QSA_F32 or QSA_BF16");
    return QSA_OK;
}

qsa_status check_workspace(const Plan &plan, void *ws, size_t bytes)
{
    if (plan.ws_bytes > 0 && (!ws || bytes < plan.ws_bytes))
        return fail(QSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", plan.ws_bytes,
                    bytes, ws ? "" : " (NULL)");
    if (plan.ws_bytes > 0 && ((uintptr_t)ws & 15u))
        return fail(QSA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    return QSA_OK;
}

qsa_status sparse_plan(const qsa_ragged_q *q, const qsa_paged_cache *kv, int64_t W,
                       const qsa_launch_options *opts, Plan *plan)
{
    qsa_status s = check_cache(kv, "kv", 2);
    if (s == QSA_OK)
        s = check_q(q, kv, true);
    if (s == QSA_OK && (W < 0 || W > (int64_t(1) << 31)))
        s = fail(QSA_ERR_SHAPE, "selection_width must be in [0, 2^31]");
    if (s == QSA_OK)
        s = plan_gather(q, kv->num_kv_heads, q->dtype, KEYS_TOKEN_INDICES, W, 1, opts, plan);
    return s;
}

qsa_status block_plan(const qsa_ragged_q *q, const qsa_paged_cache *kv, int64_t topk,
                      int64_t block_size, const qsa_launch_options *opts, Plan *plan)
{
    qsa_status s = check_cache(kv, "kv", 2);
    if (s == QSA_OK)
        s = check_q(q, kv, true);
    if (s == QSA_OK && q->dtype != QSA_BF16 && q->dtype != QSA_FP8_E4M3)
        s = fail(QSA_ERR_DTYPE, "block-sparse attention takes BF16 or FP8_E4M3 q and cache");
    if (s == QSA_OK && topk < 1)
        s = fail(QSA_ERR_SHAPE, "topk must be >= 1");
    if (s == QSA_OK && (block_size < 1 || kv->page_size % block_size != 0))
        s = fail(QSA_ERR_SHAPE, "block_size %lld must be >= 1 and divide page_size %lld",
                 (long long)block_size, (long long)kv->page_size);
    // (block_size divides page_size <= 2^30 here)
    if (s == QSA_OK && (topk > (int64_t(1) << 30) || topk * block_size > (int64_t(1) << 30)))
        s = fail(QSA_ERR_SHAPE, "topk * block_size out of range");
    if (s == QSA_OK)
        s = plan_gather(q, kv->num_kv_heads, q->dtype, KEYS_BLOCKS, topk * block_size, block_size, opts, plan);
    return s;
}

qsa_status dense_plan(const qsa_ragged_q *q, int64_t num_kv_heads, int32_t causal, int64_t window,
                      const qsa_launch_options *opts, Plan *plan)
{
    if (!q)
        return fail(QSA_ERR_NULL, "q descriptor is NULL");
    if (!q->input_row_offsets)
        return fail(QSA_ERR_NULL, "input_row_offsets is required");
    if (q->total_q < 0 || q->batch < 1 || q->num_q_heads < 1 || q->head_dim < 1)
        return fail(QSA_ERR_SHAPE, "q: total_q >= 0, batch >= 1, num_q_heads >= 1, head_dim >= 1");
    if (q->total_q > (int64_t(1) << 31) - 1 || q->batch > (int64_t(1) << 31) - 1 || q->num_q_heads > 65536)
        return fail(QSA_ERR_SHAPE, "q: total_q, batch or num_q_heads out of range");
    if (num_kv_heads < 1 || q->num_q_heads % num_kv_heads != 0)
        return fail(QSA_ERR_SHAPE, "num_q_heads %lld is not a multiple of num_kv_heads %lld",
                    (long long)q->num_q_heads, (long long)num_kv_heads);
    if (causal != 0 && causal != 1)
        return fail(QSA_ERR_SHAPE, "causal must be 0 or 1");
    if (window != -1 && window < 1)
        return fail(QSA_ERR_SHAPE, "window must be -1 (none) or >= 1");
    if (q->dtype != QSA_F32 && q->dtype != QSA_BF16 && q->dtype != QSA_FP8_E4M3)
        return fail(QSA_ERR_DTYPE, "q dtype %d is not accepted", q->dtype);
    if (q->total_q > 0 && q->max_prompt_length < 1)
        return fail(QSA_ERR_SHAPE, "max_prompt_length must be at least the longest sequence");
    int64_t cap = q->max_prompt_length;
    if (causal && window > 0 && window < cap)
        cap = window;
    return plan_gather(q, num_kv_heads, q->dtype, KEYS_DENSE, cap, 1, opts, plan);
}

qsa_status latent_plan(const qsa_ragged_q *q, int64_t window, int64_t num_comp,
                       const qsa_launch_options *opts, Plan *plan)
{
    if (!q)
        return fail(QSA_ERR_NULL, "q descriptor is NULL");
    if (window < 1)
        return fail(QSA_ERR_SHAPE, "window must be >= 1");
    if (num_comp < 0)
        return fail(QSA_ERR_SHAPE, "num_comp must be >= 0");
    if (window > (int64_t(1) << 30) || num_comp > (int64_t(1) << 30) || window + num_comp > (int64_t(1) << 30))
        return fail(QSA_ERR_SHAPE, "window + num_comp out of range");
    return plan_gather(q, 1, q->dtype, KEYS_LATENT, window + num_comp, 1, opts, plan);
}

// qsa_sparse_attention with a caller workspace, or (scratch = true) with the
// library's own device scratch in place of one.
qsa_status sparse_attention(void *out, int32_t out_dtype, const qsa_ragged_q *q, const qsa_paged_cache *kv,
                            uint32_t layer_idx, const int32_t *token_indices, int64_t selection_width,
                            const int32_t *counts, float scale, const qsa_launch_options *opts,
                            void *workspace, size_t workspace_bytes, bool scratch, void *stream)
{
    Plan plan;
    qsa_status s = sparse_plan(q, kv, selection_width, opts, &plan);
    if (s != QSA_OK)
        return s;
    if ((s = check_out(out, out_dtype, q)) != QSA_OK)
        return s;
    if (layer_idx >= kv->num_layers)
        return fail(QSA_ERR_SHAPE, "layer_idx %u >= num_layers %lld", layer_idx,
                    (long long)kv->num_layers);
    if (q->total_q > 0 && (!counts || (selection_width > 0 && !token_indices)))
        return fail(QSA_ERR_NULL, "token_indices and counts are required");
    if (!std::isfinite(scale))
        return fail(QSA_ERR_SHAPE, "scale must be finite");
    if (scratch) {
        if (plan.ws_bytes > kNoAllocScratchBytes)
            return fail(QSA_ERR_WORKSPACE, "this call needs %zu bytes of split-K scratch; the library's own "
                                           "scratch holds %zu (use fewer splits, fewer rows per call, or "
                                           "qsa_sparse_attention with a workspace)",
                        plan.ws_bytes, kNoAllocScratchBytes);
        workspace = nullptr;
        workspace_bytes = 0;
        if (plan.ws_bytes > 0 && q->total_q > 0) {
            const int err = scratch_address(&workspace);
            if (err)
                return fail(QSA_ERR_HIP, "device scratch lookup failed: %s", hip_error_text(err));
            workspace_bytes = kNoAllocScratchBytes;
        }
    } else if ((s = check_workspace(plan, workspace, workspace_bytes)) != QSA_OK) {
        return s;
    }
    GatherParams p;
    fill_common(p, out, out_dtype, q, kv->num_kv_heads, layer_idx, scale, plan, workspace);
    p.kv = cache_addr(kv, layer_idx);
    p.cache_lengths = kv->cache_lengths;
    p.list_kind = KEYS_TOKEN_INDICES;
    p.indices = token_indices;
    p.counts = counts;
    p.width = selection_width;
    return run(p, plan, stream);
}

}  // namespace

extern "C" {

qsa_status qsa_sparse_attention_workspace_size(const qsa_ragged_q *q, const qsa_paged_cache *kv,
                                               int64_t selection_width,
                                               const qsa_launch_options *opts, size_t *bytes)
{
    clear_error();
    if (!bytes)
        return fail(QSA_ERR_NULL, "bytes is NULL");
    Plan plan;
    qsa_status s = sparse_plan(q, kv, selection_width, opts, &plan);
    *bytes = s == QSA_OK ? plan.ws_bytes : 0;
    return s;
}

qsa_status qsa_sparse_attention(void *out, int32_t out_dtype, const qsa_ragged_q *q,
                                const qsa_paged_cache *kv, uint32_t layer_idx,
                                const int32_t *token_indices, int64_t selection_width,
                                const int32_t *counts, float scale,
                                const qsa_launch_options *opts, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    clear_error();
    return sparse_attention(out, out_dtype, q, kv, layer_idx, token_indices, selection_width, counts, scale,
                            opts, workspace, workspace_bytes, false, stream);
}

qsa_status qsa_sparse_attention_no_alloc(void *out, int32_t out_dtype, const qsa_ragged_q *q,
                                         const qsa_paged_cache *kv, uint32_t layer_idx,
                                         const int32_t *token_indices, int64_t selection_width,
                                         const int32_t *counts, float scale,
                                         const qsa_launch_options *opts, void *stream)
{
    clear_error();
    return sparse_attention(out, out_dtype, q, kv, layer_idx, token_indices, selection_width, counts, scale,
                            opts, nullptr, 0, true, stream);
}

qsa_status qsa_block_sparse_attention_workspace_size(const qsa_ragged_q *q, const qsa_paged_cache *kv,
                                                     int64_t topk, int64_t block_size,
                                                     const qsa_launch_options *opts, size_t *bytes)
{
    clear_error();
    if (!bytes)
        return fail(QSA_ERR_NULL, "bytes is NULL");
    Plan plan;
    qsa_status s = block_plan(q, kv, topk, block_size, opts, &plan);
    *bytes = s == QSA_OK ? plan.ws_bytes : 0;
    return s;
}

qsa_status qsa_block_sparse_attention(void *out, const qsa_ragged_q *q, const qsa_paged_cache *kv,
                                      uint32_t layer_idx, const int32_t *d_indices, int64_t topk,
                                      int64_t block_size, float scale,
                                      const uint32_t *cache_row_offsets,
                                      const uint32_t *msa_scalar_args,
                                      const qsa_launch_options *opts, void *workspace,
                                      size_t workspace_bytes, void *stream)
{
    (void)cache_row_offsets;
    (void)msa_scalar_args;
    clear_error();
    Plan plan;
    qsa_status s = block_plan(q, kv, topk, block_size, opts, &plan);
    if (s != QSA_OK)
        return s;
    if ((s = check_out(out, QSA_BF16, q)) != QSA_OK)
        return s;
    if (layer_idx >= kv->num_layers)
        return fail(QSA_ERR_SHAPE, "layer_idx %u >= num_layers %lld", layer_idx,
                    (long long)kv->num_layers);
    if (q->total_q > 0 && !d_indices)
        return fail(QSA_ERR_NULL, "d_indices is required");
    if (!std::isfinite(scale))
        return fail(QSA_ERR_SHAPE, "scale must be finite");
    if ((s = check_workspace(plan, workspace, workspace_bytes)) != QSA_OK)
        return s;
    GatherParams p;
    fill_common(p, out, QSA_BF16, q, kv->num_kv_heads, layer_idx, scale, plan, workspace);
    p.kv = cache_addr(kv, layer_idx);
    p.cache_lengths = kv->cache_lengths;
    p.list_kind = KEYS_BLOCKS;
    p.block_size = (int32_t)block_size;
    p.block_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctzll((unsigned long long)block_size) : -1;
    p.indices = d_indices;
    p.width = topk;
    return run(p, plan, stream);
}

qsa_status qsa_latent_sparse_attention_workspace_size(const qsa_ragged_q *q, int64_t window,
                                                      int64_t num_comp,
                                                      const qsa_launch_options *opts,
                                                      size_t *bytes)
{
    clear_error();
    if (!bytes)
        return fail(QSA_ERR_NULL, "bytes is NULL");
    Plan plan;
    qsa_status s = latent_plan(q, window, num_comp, opts, &plan);
    *bytes = s == QSA_OK ? plan.ws_bytes : 0;
    return s;
}

qsa_status qsa_latent_sparse_attention(void *out, int32_t out_dtype, const qsa_ragged_q *q,
                                       const qsa_paged_cache *swa, const qsa_paged_cache *comp,
                                       uint32_t layer_idx, int64_t window,
                                       const int32_t *comp_indices, int64_t num_comp,
                                       const float *attn_sink, float scale,
                                       const qsa_launch_options *opts, void *workspace,
                                       size_t workspace_bytes, void *stream)
{
    clear_error();
    qsa_status s = check_cache(swa, "swa", 1);
    if (s == QSA_OK)
        s = check_cache(comp, "comp", 1);
    if (s != QSA_OK)
        return s;
    if (swa->num_kv_heads != 1 || comp->num_kv_heads != 1)
        return fail(QSA_ERR_SHAPE, "latent leaves hold one head (num_kv_heads must be 1)");
    if (comp->dtype != swa->dtype || comp->head_dim != swa->head_dim)
        return fail(QSA_ERR_SHAPE, "swa and comp leaves must share dtype and head_dim");
    if ((s = check_q(q, swa, false)) != QSA_OK)
        return s;
    Plan plan;
    if ((s = latent_plan(q, window, num_comp, opts, &plan)) != QSA_OK)
        return s;
    if ((s = check_out(out, out_dtype, q)) != QSA_OK)
        return s;
    if (layer_idx >= swa->num_layers || layer_idx >= comp->num_layers)
        return fail(QSA_ERR_SHAPE, "layer_idx %u out of range", layer_idx);
    if (q->total_q > 0 && ((num_comp > 0 && !comp_indices) || !attn_sink))
        return fail(QSA_ERR_NULL, "comp_indices and attn_sink are required");
    if (!std::isfinite(scale))
        return fail(QSA_ERR_SHAPE, "scale must be finite");
    if ((s = check_workspace(plan, workspace, workspace_bytes)) != QSA_OK)
        return s;
    GatherParams p;
    fill_common(p, out, out_dtype, q, 1, layer_idx, scale, plan, workspace);
    p.kv = cache_addr(swa, layer_idx);
    p.comp = cache_addr(comp, layer_idx);
    p.cache_lengths = swa->cache_lengths;
    p.list_kind = KEYS_LATENT;
    p.indices = comp_indices;
    p.width = num_comp;
    p.window = window;
    p.sink = attn_sink;
    return run(p, plan, stream);
}

const char *qsa_last_error(void) { return last_error_text(); }

int32_t qsa_abi_version(void) { return QSA_ABI_VERSION; }

size_t qsa_struct_size(int32_t which)
{
    switch (which) {
    case 0: return sizeof(qsa_paged_cache);
    case 1: return sizeof(qsa_ragged_q);
    case 2: return sizeof(qsa_launch_options);
    default: return 0;
    }
}

qsa_status qsa_ragged_attention_workspace_size(const qsa_ragged_q *q, int64_t num_kv_heads, int32_t causal,
                                               int64_t window, const qsa_launch_options *opts, size_t *bytes)
{
    clear_error();
    if (!bytes)
        return fail(QSA_ERR_NULL, "bytes is NULL");
    Plan plan;
    qsa_status s = dense_plan(q, num_kv_heads, causal, window, opts, &plan);
    *bytes = s == QSA_OK ? plan.ws_bytes : 0;
    return s;
}

qsa_status qsa_ragged_attention(void *out, int32_t out_dtype, const qsa_ragged_q *q, const void *k,
                                const void *v, int64_t num_kv_heads, int32_t causal, int64_t window,
                                float scale, const qsa_launch_options *opts, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    clear_error();
    Plan plan;
    qsa_status s = dense_plan(q, num_kv_heads, causal, window, opts, &plan);
    if (s != QSA_OK)
        return s;
    if ((s = check_out(out, out_dtype, q)) != QSA_OK)
        return s;
    if (q->total_q > 0 && (!q->q || !k || !v))
        return fail(QSA_ERR_NULL, "q, k and v are required");
    if (q->total_q > 0 && (!aligned16(q->q) || !aligned16(k) || !aligned16(v)))
        return fail(QSA_ERR_SHAPE, "q, k and v must be 16-byte aligned");
    if (!std::isfinite(scale))
        return fail(QSA_ERR_SHAPE, "scale must be finite");
    if ((s = check_workspace(plan, workspace, workspace_bytes)) != QSA_OK)
        return s;
    GatherParams p;
    fill_common(p, out, out_dtype, q, num_kv_heads, 0, scale, plan, workspace);
    p.list_kind = KEYS_DENSE;
    p.dense_k = k;
    p.dense_v = v;
    p.dense_causal = causal;
    p.window = window > 0 ? window : 0;
    // matrix-core groups without a split: workgroups of consecutive rows share key tiles
    // (unless a launch option asks for a wavefront count, which only the per-row kernel takes)
    if (plan.path == PATH_MFMA && plan.num_splits == 1 &&
        (!opts || opts->waves == 0) && mfma_flash_supported(q->dtype, p.group, p.head_dim)) {
        if (q->total_q == 0)
            return QSA_OK;
        int err = 0;
        if (t_ev_start && t_ev_stop)
            err = record_event(t_ev_start, stream);
        if (!err)
            err = launch_gather_mfma_flash(p, stream);
        if (!err && t_ev_start && t_ev_stop)
            err = record_event(t_ev_stop, stream);
        if (err)
            return fail(QSA_ERR_HIP, "HIP launch failed: %s", hip_error_text(err));
        return QSA_OK;
    }
    return run(p, plan, stream);
}

qsa_status qsa_compress_keys(void *block_keys, int64_t max_blocks, const void *gamma, const void *freqs_cis,
                             int32_t freq_dtype, int64_t num_positions, int64_t rotary_dim,
                             const int32_t *key_counts, const qsa_paged_cache *kv, int64_t batch,
                             uint32_t layer_idx, uint32_t max_prompt_length, int64_t ratio, float eps,
                             void *stream)
{
    clear_error();
    qsa_status s = check_cache(kv, "kv", 2);
    if (s != QSA_OK)
        return s;
    if (kv->num_kv_heads != 1)
        return fail(QSA_ERR_SHAPE, "the indexer cache holds one head (num_kv_heads must be 1)");
    if (!compress_supported(kv->dtype, (int32_t)std::min<int64_t>(kv->head_dim, 1 << 20)))
        return fail(kv->dtype == QSA_F32 || kv->dtype == QSA_BF16 ? QSA_ERR_UNSUPPORTED : QSA_ERR_DTYPE,
                    "key compression takes F32 or BF16 keys whose rows are 16, 32, 64, ... or 1024 bytes "
                    "(dtype %d, head_dim %lld)", kv->dtype, (long long)kv->head_dim);
    if (layer_idx >= (uint64_t)kv->num_layers)
        return fail(QSA_ERR_SHAPE, "layer_idx %u >= num_layers %lld", layer_idx, (long long)kv->num_layers);
    if (batch < 0 || batch > (int64_t(1) << 31) - 1 || max_blocks < 0)
        return fail(QSA_ERR_SHAPE, "batch and max_blocks must be >= 0 (batch < 2^31)");
    if (ratio < 1 || ratio > (int64_t(1) << 30))
        return fail(QSA_ERR_SHAPE, "ratio must be >= 1");
    if (rotary_dim < 0 || rotary_dim % 2 || rotary_dim > kv->head_dim)
        return fail(QSA_ERR_SHAPE, "rotary_dim %lld must be even and within [0, head_dim %lld]",
                    (long long)rotary_dim, (long long)kv->head_dim);
    if (freq_dtype != QSA_F32 && freq_dtype != QSA_BF16)
        return fail(QSA_ERR_DTYPE, "freq_dtype must be QSA_F32 or QSA_BF16");
    if (!std::isfinite(eps) || eps < 0.f)
        return fail(QSA_ERR_SHAPE, "eps must be finite and >= 0");
    // blocks per sequence the launch covers: the row stride, the keys the step can hold
    // (max_cache_length + max_prompt_length, when given) and the positions the page
    // table (and 31-bit positions) can address
    int64_t bound = max_blocks;
    // (a max_cache_length of 0 says nothing about the cache: no bound from the hint then)
    const int64_t hint = (int64_t)kv->max_cache_length + (int64_t)max_prompt_length;
    if (kv->max_cache_length > 0)
        bound = std::min(bound, hint / ratio);
    const int64_t addressable = std::min(kv->max_pages * kv->page_size, (int64_t(1) << 31) - 1);
    bound = std::min(bound, addressable / ratio);
    if (batch == 0 || bound == 0)
        return QSA_OK;
    if (!block_keys || !gamma || !key_counts)
        return fail(QSA_ERR_NULL, "block_keys, gamma and key_counts are required");
    if (!aligned16(block_keys) || !aligned16(gamma))
        return fail(QSA_ERR_SHAPE, "block_keys and gamma must be 16-byte aligned");
    if (rotary_dim > 0) {
        if (!freqs_cis)
            return fail(QSA_ERR_NULL, "freqs_cis is required when rotary_dim > 0");
        if (((uintptr_t)freqs_cis & (freq_dtype == QSA_F32 ? 7u : 3u)) != 0)
            return fail(QSA_ERR_SHAPE, "freqs_cis must be aligned to one (cos, sin) pair");
        if (num_positions < 0 || (bound - 1) * ratio >= num_positions)
            return fail(QSA_ERR_SHAPE, "freqs_cis has %lld positions; blocks up to %lld start at position %lld",
                        (long long)num_positions, (long long)bound, (long long)((bound - 1) * ratio));
    }
    const int64_t per_wg = kCompressThreads / compress_team_lanes(kv->dtype == QSA_F32 ? 4 : 2, (int)kv->head_dim);
    if (batch * ((bound + per_wg - 1) / per_wg) > (int64_t(1) << 31) - 1)
        return fail(QSA_ERR_SHAPE, "batch * max_blocks out of range");
    CompressParams p;
    std::memset(&p, 0, sizeof p);
    p.out = block_keys;
    p.gamma = gamma;
    p.freqs = freqs_cis;
    p.key_counts = key_counts;
    p.kv = cache_addr(kv, layer_idx);
    p.max_blocks = max_blocks;
    p.blocks_bound = bound;
    p.dtype = kv->dtype;
    p.freq_dtype = freq_dtype;
    p.head_dim = (int32_t)kv->head_dim;
    p.rotary_dim = (int32_t)rotary_dim;
    p.ratio = (int32_t)ratio;
    p.batch = (int32_t)batch;
    p.eps = eps;
    int err = 0;
    if (t_ev_start && t_ev_stop)
        err = record_event(t_ev_start, stream);
    if (!err)
        err = launch_compress_keys(p, stream);
    if (!err && t_ev_start && t_ev_stop)
        err = record_event(t_ev_stop, stream);
    if (err)
        return fail(QSA_ERR_HIP, "HIP launch failed: %s", hip_error_text(err));
    return QSA_OK;
}

// Candidate blocks per row a selection launch covers (0 when none).
static int64_t select_bound(int64_t max_blocks, int64_t ratio, uint32_t max_cache_length, uint32_t max_prompt_length)
{
    int64_t bound = max_blocks;
    // the hint bounds the candidates only when it describes the cache (a max_cache_length
    // of 0 gives no bound: the candidates are then limited by max_blocks alone)
    const int64_t hint = (int64_t)max_cache_length + (int64_t)max_prompt_length;
    if (max_cache_length > 0 && hint / ratio < bound)
        bound = hint / ratio;
    return bound;
}

static qsa_status select_check(const qsa_ragged_q *q, int64_t max_blocks, int64_t ratio, int64_t topk,
                               uint32_t max_cache_length, int64_t *bound)
{
    if (!q)
        return fail(QSA_ERR_NULL, "q_index descriptor is NULL");
    if (!q->input_row_offsets)
        return fail(QSA_ERR_NULL, "input_row_offsets is required");
    if (q->total_q < 0 || q->batch < 1 || q->num_q_heads != 1 || q->head_dim < 1)
        return fail(QSA_ERR_SHAPE, "q_index: total_q >= 0, batch >= 1, one head, head_dim >= 1");
    if (q->total_q > (int64_t(1) << 31) - 1 || q->batch > (int64_t(1) << 31) - 1)
        return fail(QSA_ERR_SHAPE, "q_index: total_q or batch out of range");
    if (!select_supported(q->dtype, (int32_t)std::min<int64_t>(q->head_dim, 1 << 20)))
        return fail(q->dtype == QSA_F32 || q->dtype == QSA_BF16 ? QSA_ERR_UNSUPPORTED : QSA_ERR_DTYPE,
                    "block selection takes F32 or BF16 queries and keys whose rows are 16, 32, 64, ... or "
                    "1024 bytes (dtype %d, head_dim %lld)", q->dtype, (long long)q->head_dim);
    if (ratio < 1 || ratio > (int64_t(1) << 20) || topk < 0 || topk > (int64_t(1) << 24) || max_blocks < 0)
        return fail(QSA_ERR_SHAPE, "ratio >= 1, topk >= 0 and max_blocks >= 0 are required");
    *bound = select_bound(max_blocks, ratio, max_cache_length, q->max_prompt_length);
    if (*bound > kSelectMaxCandidates)
        return fail(QSA_ERR_UNSUPPORTED, "at most %lld candidate blocks per row (max_blocks, or (max_cache_length "
                                         "+ max_prompt_length) / ratio when max_cache_length > 0, is %lld)",
                    (long long)kSelectMaxCandidates, (long long)*bound);
    if (q->total_q * ((*bound + 15) / 16) > (int64_t(1) << 31) - 1)
        return fail(QSA_ERR_SHAPE, "total_q * candidate blocks out of range");
    return QSA_OK;
}

qsa_status qsa_select_blocks_workspace_size(const qsa_ragged_q *q_index, int64_t max_blocks, int64_t ratio,
                                            int64_t topk, uint32_t max_cache_length, size_t *bytes)
{
    clear_error();
    if (!bytes)
        return fail(QSA_ERR_NULL, "bytes is NULL");
    *bytes = 0;
    int64_t bound;
    qsa_status s = select_check(q_index, max_blocks, ratio, topk, max_cache_length, &bound);
    if (s == QSA_OK)
        *bytes = (size_t)q_index->total_q * (size_t)bound * sizeof(float);
    return s;
}

qsa_status qsa_select_blocks(int32_t *token_indices, int64_t selection_width, int32_t *counts, int32_t *blocks,
                             const qsa_ragged_q *q_index, const void *block_keys, int64_t max_blocks,
                             const uint32_t *cache_lengths, uint32_t max_cache_length, int64_t ratio, int64_t topk,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    clear_error();
    int64_t bound;
    qsa_status s = select_check(q_index, max_blocks, ratio, topk, max_cache_length, &bound);
    if (s != QSA_OK)
        return s;
    if (selection_width < topk * ratio + ratio - 1)
        return fail(QSA_ERR_SHAPE, "selection_width %lld cannot hold topk * ratio + ratio - 1 = %lld positions",
                    (long long)selection_width, (long long)(topk * ratio + ratio - 1));
    if (q_index->total_q == 0)
        return QSA_OK;
    if (!token_indices || !counts || !cache_lengths || !q_index->q || (bound > 0 && !block_keys))
        return fail(QSA_ERR_NULL, "token_indices, counts, cache_lengths, q_index and block_keys are required");
    if (!aligned16(q_index->q) || (bound > 0 && !aligned16(block_keys)))
        return fail(QSA_ERR_SHAPE, "q_index and block_keys must be 16-byte aligned");
    const size_t need = (size_t)q_index->total_q * (size_t)bound * sizeof(float);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(QSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (need > 0 && ((uintptr_t)workspace & 15u))
        return fail(QSA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    SelectParams p;
    std::memset(&p, 0, sizeof p);
    p.token_indices = token_indices;
    p.counts = counts;
    p.blocks = topk > 0 ? blocks : nullptr;
    p.q_index = q_index->q;
    p.block_keys = block_keys;
    p.row_off = q_index->input_row_offsets;
    p.cache_lengths = cache_lengths;
    p.scores = static_cast<float *>(workspace);
    p.total_q = q_index->total_q;
    p.width = selection_width;
    p.max_blocks = max_blocks;
    p.cand_bound = bound;
    p.batch = (int32_t)q_index->batch;
    p.dtype = q_index->dtype;
    p.head_dim = (int32_t)q_index->head_dim;
    p.ratio = (int32_t)ratio;
    p.topk = (int32_t)topk;
    const bool timed = t_ev_start && t_ev_stop;
    int err = launch_select_blocks(p, stream, timed ? t_ev_start : nullptr, timed ? t_ev_stop : nullptr);
    if (err)
        return fail(QSA_ERR_HIP, "HIP launch failed: %s", hip_error_text(err));
    return QSA_OK;
}

qsa_status qsa_stream_read(const void *src, size_t bytes, uint32_t *sink, uint32_t grid, void *stream)
{
    clear_error();
    if (grid < 1 || grid > (1u << 20))
        return fail(QSA_ERR_SHAPE, "grid must be in [1, 2^20]");
    if (!sink || (bytes > 0 && !src))
        return fail(QSA_ERR_NULL, "src and sink are required");
    if (!aligned16(src) || bytes % 16 != 0)
        return fail(QSA_ERR_SHAPE, "src must be 16-byte aligned and bytes a multiple of 16");
    const int err = launch_stream_read(src, bytes, sink, grid, stream);
    if (err)
        return fail(QSA_ERR_HIP, "HIP launch failed: %s", hip_error_text(err));
    return QSA_OK;
}

qsa_status qsa_gather_replay(const void *base, uint64_t region_bytes, const int64_t *offsets, const int32_t *counts,
                             uint32_t items, uint32_t max_keys, uint32_t row_bytes, int64_t plane_delta,
                             uint32_t *sink, void *stream)
{
    clear_error();
    if (row_bytes != 64 && row_bytes != 128 && row_bytes != 256 && row_bytes != 512 && row_bytes != 1024)
        return fail(QSA_ERR_SHAPE, "row_bytes must be 64, 128, 256, 512 or 1024");
    if (max_keys < 1 || max_keys > (1u << 20))
        return fail(QSA_ERR_SHAPE, "max_keys must be in [1, 2^20]");
    if (items > 0x7fffffffu)
        return fail(QSA_ERR_SHAPE, "items must be below 2^31");
    if (items > 0 && (!base || !offsets || !counts || !sink))
        return fail(QSA_ERR_NULL, "base, offsets, counts and sink are required");
    if (!aligned16(base) || plane_delta % 16 != 0)
        return fail(QSA_ERR_SHAPE, "base must be 16-byte aligned and plane_delta a multiple of 16");
    if (items > 0 && region_bytes < row_bytes)
        return fail(QSA_ERR_SHAPE, "region_bytes must hold at least one row");
    const int err = launch_gather_replay(base, region_bytes, offsets, counts, items, max_keys, row_bytes,
                                         plane_delta, sink, stream);
    if (err)
        return fail(QSA_ERR_HIP, "HIP launch failed: %s", hip_error_text(err));
    return QSA_OK;
}

void qsa_set_timing_events(void *start, void *stop)
{
    t_ev_start = start;
    t_ev_stop = stop;
}

}  // extern "C"
