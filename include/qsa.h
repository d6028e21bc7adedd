/*
 * qsa.h - C ABI of the MI355X (gfx950) sparse paged attention library.
 *
 * Three operations over a ragged batch of query rows and a paged KV cache, and the
 * dense ragged attention they are compared with:
 *
 *   qsa_sparse_attention         index-selected sparse GQA: every query row attends
 *                                to the positions its token_indices row lists
 *                                ("QSASparseAttentionRaggedPaged", summary, Tensor
 *                                shapes and execute() Args);
 *   qsa_block_sparse_attention   block-sparse attention over top-k KV blocks per
 *                                (kv head, query row) ("Struct_msa_attention_ragged_paged",
 *                                design notes and Args);
 *   qsa_latent_sparse_attention  one shared latent head: sliding-window keys plus
 *                                listed compressed entries plus a per-head sink logit
 *                                ("latent_sparse_attention_ragged_paged", summary,
 *                                Parameters and Args);
 *   qsa_ragged_attention         dense causal / sliding-window / unmasked attention
 *                                over ragged q, k, v without a cache
 *                                ("RaggedFlashAttentionGPU", summary, Parameters and Args);
 *
 * and the steps that produce a selection: the key compression that pools raw index
 * keys into block keys (qsa_compress_keys, "QSACompressKeysPaged") and the top-k block
 * selection that turns them into token_indices and counts (qsa_select_blocks).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless a comment says (host). The caller owns
 *     every buffer; the library writes only the call's output buffers (`out`,
 *     `block_keys`, `token_indices`, `counts`, `blocks`) and `workspace`, never
 *     allocates, frees or synchronises, and reads no device data on the host.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   - Workspace: the size the matching *_workspace_size call reports, 16-byte
 *     aligned, contents undefined on entry (every byte a call reads there it has
 *     written earlier in the same call). Calls that share a workspace must be ordered
 *     (one stream, or synchronised); calls on different workspaces may overlap.
 *   - Arguments are checked on the host before anything is launched; a failed
 *     check returns a non-zero qsa_status and qsa_last_error() describes it. (Where
 *     the pages' ops raise an error for operand shapes that contradict their
 *     parameters - "QSASparseAttentionRaggedPaged", Raises - this library returns
 *     a status code instead.)
 *   - Row r of sequence b (input_row_offsets[b] <= r < input_row_offsets[b+1]) is
 *     at position cache_lengths[b] + (r - input_row_offsets[b]); the cache already
 *     holds positions 0 .. that position. Only block-sparse (causal clip) and latent
 *     (window) use the position.
 *   - Query head h reads kv head h / (num_q_heads / num_kv_heads).
 *   - Device-data contract (not checked on the host): positions and page ids must
 *     address the cache. The kernels never dereference an entry that does not
 *     (a position outside [0, max_pages * page_size), a page id >= num_pages): such
 *     an entry is skipped as if it were not listed.
 *   - Results are exact softmax attention up to fp32 rounding: fp32 accumulation,
 *     fp32 or bf16 (round to nearest even) output. A row with no keys is all zeros.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 5

/* Element types. QSA_FP8_E4M3 is the OCP 8-bit E4M3 "fn" format (bias 7, max 448,
 * no infinity), scale-free as the block-sparse page states for its FP8 path. */
typedef enum { QSA_F32 = 0, QSA_BF16 = 1, QSA_FP8_E4M3 = 2 } qsa_dtype;

typedef enum {
    QSA_OK = 0,
    QSA_ERR_NULL = 1,        /* a required pointer is NULL */
    QSA_ERR_SHAPE = 2,       /* shapes disagree with each other or with the parameters */
    QSA_ERR_DTYPE = 3,       /* element types disagree or are not accepted here */
    QSA_ERR_UNSUPPORTED = 4, /* valid but not built: (dtype, group, head_dim) or launch option */
    QSA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than *_workspace_size reports */
    QSA_ERR_HIP = 6          /* the HIP runtime refused a launch */
} qsa_status;

/* One paged cache leaf ("QSASparseAttentionRaggedPaged" Tensor shapes / Args:
 * kv_blocks, page_stride, cache_lengths, kv_lookup_table, max_cache_length). */
typedef struct {
    const void *blocks;      /* [num_pages, num_planes, num_layers, page_size, num_kv_heads, head_dim] */
    int32_t dtype;           /* qsa_dtype */
    int32_t reserved0;
    int64_t num_pages;
    int64_t num_planes;      /* 2 = K and V planes; 1 = latent leaf (the row is key and value) */
    int64_t num_layers;
    int64_t page_size;
    int64_t num_kv_heads;
    int64_t head_dim;
    int64_t page_stride;     /* elements from one page to the next; -1 = packed.  The inside of a
                                page is always packed [num_planes, num_layers, page_size, Hkv, D]. */
    const uint32_t *lookup_table; /* [batch, max_pages]: physical page of each logical page */
    int64_t max_pages;
    const uint32_t *cache_lengths; /* [batch]: keys cached before this step's rows */
    uint32_t max_cache_length;     /* (host) max of cache_lengths, or 0 when not known; a sizing
                                      hint (0 bounds nothing) */
    uint32_t reserved1;
} qsa_paged_cache;

/* Ragged query rows ("QSASparseAttentionRaggedPaged": q, input_row_offsets,
 * max_prompt_length). */
typedef struct {
    const void *q;           /* [total_q, num_q_heads, head_dim], rows contiguous */
    int32_t dtype;           /* qsa_dtype; must equal the cache's */
    int32_t reserved0;
    int64_t total_q;
    int64_t num_q_heads;
    int64_t head_dim;
    int64_t batch;
    const uint32_t *input_row_offsets; /* [batch + 1], non-decreasing, last = total_q */
    uint32_t max_prompt_length;        /* (host) max rows of one sequence; a sizing hint only */
    uint32_t reserved1;
} qsa_ragged_q;

/* Launch knobs ("QSASparseAttentionRaggedPaged" execute Parameters: warps per CTA
 * and keys in flight). Pass NULL, or zeros, for the library's choice. */
typedef struct {
    int32_t num_splits;      /* split-K partitions of each row's key list; 0 = automatic */
    int32_t waves;           /* wavefronts per workgroup; 0 = automatic */
    int32_t unroll;          /* gathered keys a key team has in flight; 0 = automatic */
    int32_t reserved;        /* must be 0 */
} qsa_launch_options;

/* ------------------------------------------------------------------------- */
/* Index-selected sparse GQA ("QSASparseAttentionRaggedPaged").
 *
 * out[r, h, :] = softmax_j(scale * q[r,h,:] . K_j) . V_j over the first
 * n = min(counts[r], selection_width) entries j of token_indices[r, :], where
 * position p = token_indices[r, j] of r's sequence is read at page
 * kv_lookup_table[b, p / page_size], slot p % page_size, plane 0 (K) or 1 (V),
 * layer layer_idx, kv head h / group. Entries at or past counts[r] are never read.
 *
 *   out            [total_q, num_q_heads, head_dim] of out_dtype (QSA_F32 or QSA_BF16)
 *   q, kv          q->dtype == kv->dtype, in {F32, BF16, FP8_E4M3}; kv->num_planes == 2
 *   token_indices  [total_q, selection_width] int32, positions within each row's sequence
 *   counts         [total_q] int32; <= 0 gives a zero row, > selection_width is clamped
 *   workspace      >= qsa_sparse_attention_workspace_size(...) bytes (may be NULL when that is 0)
 * Supported now: group in {1, 2, 4} with head_dim in {64, 128, 256} (wavefront dot
 * products), group in {8, 16} with head_dim 128 (matrix cores).
 */
qsa_status qsa_sparse_attention_workspace_size(const qsa_ragged_q *q, const qsa_paged_cache *kv,
                                               int64_t selection_width,
                                               const qsa_launch_options *opts, size_t *bytes);

qsa_status qsa_sparse_attention(void *out, int32_t out_dtype, const qsa_ragged_q *q,
                                const qsa_paged_cache *kv, uint32_t layer_idx,
                                const int32_t *token_indices, int64_t selection_width,
                                const int32_t *counts, float scale,
                                const qsa_launch_options *opts, void *workspace,
                                size_t workspace_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): qsa_sparse_attention without a workspace.
 * Same arguments, checks, kernels and results as qsa_sparse_attention with the same
 * options; the split-K partials (when the plan splits) go to a device array the
 * library holds, QSA_NO_ALLOC_SCRATCH_BYTES on every GPU it runs on, from when the
 * library's code is loaded there until the process ends. The call allocates and frees
 * nothing. A call whose plan needs more scratch than that returns QSA_ERR_WORKSPACE
 * before any launch (fewer splits or fewer rows per call fit). All calls on one GPU
 * share its array: calls that can overlap on one GPU (different streams, or several
 * threads) race and give undefined results; order them on one stream. The device
 * current on the calling thread must be the one `stream` belongs to. Nothing in the
 * array carries over from one call to the next. */
#define QSA_NO_ALLOC_SCRATCH_BYTES ((size_t)16 << 20)

qsa_status qsa_sparse_attention_no_alloc(void *out, int32_t out_dtype, const qsa_ragged_q *q,
                                         const qsa_paged_cache *kv, uint32_t layer_idx,
                                         const int32_t *token_indices, int64_t selection_width,
                                         const int32_t *counts, float scale,
                                         const qsa_launch_options *opts, void *stream);

/* ------------------------------------------------------------------------- */
/* Block-sparse top-k attention ("Struct_msa_attention_ragged_paged").
 *
 * For row r at position pos and kv head g the keys are the positions
 * block_size * t + i (0 <= i < block_size) of every listed block t in
 * d_indices[g, r, 0:topk] that are <= pos; each q head of group g attends to them.
 *
 *   out        [total_q, num_q_heads, head_dim] bf16 (always, as the page states)
 *   q, kv      BF16 or FP8_E4M3, same type; FP32 accumulation; no dequant scales
 *   d_indices  [num_kv_heads, total_q, topk] int32 block ids
 *   block_size must divide kv->page_size
 *   cache_row_offsets, msa_scalar_args: optional (may be NULL) hints from the page's
 *   argument list; the result does not depend on them.
 */
qsa_status qsa_block_sparse_attention_workspace_size(const qsa_ragged_q *q, const qsa_paged_cache *kv,
                                                     int64_t topk, int64_t block_size,
                                                     const qsa_launch_options *opts, size_t *bytes);

qsa_status qsa_block_sparse_attention(void *out, const qsa_ragged_q *q, const qsa_paged_cache *kv,
                                      uint32_t layer_idx, const int32_t *d_indices, int64_t topk,
                                      int64_t block_size, float scale,
                                      const uint32_t *cache_row_offsets,
                                      const uint32_t *msa_scalar_args,
                                      const qsa_launch_options *opts, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------- */
/* Latent window + compressed + sink attention ("latent_sparse_attention_ragged_paged").
 *
 * Row r at position pos (from swa->cache_lengths) attends to the window rows at
 * positions max(0, pos - window + 1) .. pos of the token-paged leaf `swa` and to the
 * compressed rows at entries comp_indices[r, t] >= 0 of the entry-paged leaf `comp`
 * (-1 marks an unused slot, anywhere in the row). Each latent row is both key and
 * value. Head h adds attn_sink[h] (not multiplied by scale) to the softmax
 * denominator with a zero value row.
 *
 *   out           [total_q, num_q_heads, head_dim] of out_dtype (F32 or BF16)
 *   swa, comp     num_planes == 1, num_kv_heads == 1, head_dim == q->head_dim, same dtype as q
 *   comp_indices  [total_q, num_comp] int32
 *   attn_sink     [num_q_heads] float32 (-inf = no sink for that head)
 */
qsa_status qsa_latent_sparse_attention_workspace_size(const qsa_ragged_q *q, int64_t window,
                                                      int64_t num_comp,
                                                      const qsa_launch_options *opts,
                                                      size_t *bytes);

qsa_status qsa_latent_sparse_attention(void *out, int32_t out_dtype, const qsa_ragged_q *q,
                                       const qsa_paged_cache *swa, const qsa_paged_cache *comp,
                                       uint32_t layer_idx, int64_t window,
                                       const int32_t *comp_indices, int64_t num_comp,
                                       const float *attn_sink, float scale,
                                       const qsa_launch_options *opts, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------- */
/* Dense ragged attention without a KV cache ("RaggedFlashAttentionGPU": summary,
 * Parameters and Args), the dense comparison for the sparse operations above.
 *
 * Row r, the i-th row of its sequence b (L = input_row_offsets[b+1] -
 * input_row_offsets[b] rows), attends to the rows i' of the same sequence with
 * i' <= i when causal (every i' < L when not) and i' >= i - window + 1 when
 * window > 0; key i' is k[input_row_offsets[b] + i', h / group, :], value likewise.
 *
 *   out      [total_q, num_q_heads, head_dim] of out_dtype (QSA_F32 or QSA_BF16)
 *   q        q->dtype in {F32, BF16, FP8_E4M3}; q->max_prompt_length (host) must be at
 *            least the longest sequence (the pages' q_max_seq_len; it sizes the
 *            split plan, and keys past it would not be visited)
 *   k, v     [total_q, num_kv_heads, head_dim] of q->dtype, 16-byte aligned
 *   causal   0 (no mask) or 1 (causal)
 *   window   -1 for none, else >= 1 (the pages' local_window_size)
 * Supported: the same (dtype, group, head_dim) as qsa_sparse_attention; groups of
 * more than 16 are not built here.
 */
qsa_status qsa_ragged_attention_workspace_size(const qsa_ragged_q *q, int64_t num_kv_heads, int32_t causal,
                                               int64_t window, const qsa_launch_options *opts,
                                               size_t *bytes);

qsa_status qsa_ragged_attention(void *out, int32_t out_dtype, const qsa_ragged_q *q, const void *k,
                                const void *v, int64_t num_kv_heads, int32_t causal, int64_t window,
                                float scale, const qsa_launch_options *opts, void *workspace,
                                size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------- */
/* Key compression ("QSACompressKeysPaged": summary, Tensor shapes, execute Parameters
 * and Args): pools the raw index keys of a paged indexer cache into dense block keys,
 * the keys that block selection scores.
 *
 * Sequence b holds key_counts[b] raw keys (cache_lengths[b] plus this step's rows) at
 * positions 0.. of plane 0, kv head 0, layer layer_idx of `kv`. Its complete groups of
 * `ratio` consecutive keys give n_b = min(key_counts[b] / ratio, max_blocks) block keys;
 * block j (raw positions j*ratio .. j*ratio + ratio - 1) is
 *   x   = the mean of the group's raw keys,
 *   y_d = gamma_d * x_d / sqrt(mean over d of x_d^2 + eps),
 *   and for each channel pair (2i, 2i+1) with 2i + 1 < rotary_dim, with (c, s) =
 *   freqs_cis[j*ratio, 2i : 2i+2]: (c*y_2i - s*y_2i+1, s*y_2i + c*y_2i+1);
 *   channels at or past rotary_dim stay y_d.
 * (The pages name the pooling, the RMS norm and the rotary table but fix neither the
 * pooling operator nor the order nor the pairing: these are this library's readings.)
 * Block key j of sequence b is row b * max_blocks + j of block_keys. A trailing partial
 * group gives no block key, and rows at or past n_b are not written (they keep what
 * the caller left there).
 *
 *   block_keys    [batch * max_blocks, head_dim] of kv->dtype (F32 or BF16), 16-byte aligned
 *   gamma         [head_dim] of kv->dtype (the key RMS-norm weight), 16-byte aligned
 *   freqs_cis     [num_positions, rotary_dim] of freq_dtype (F32 or BF16): row p holds
 *                 rotary_dim / 2 (cos, sin) pairs; may be NULL when rotary_dim == 0
 *   key_counts    [batch] int32; <= 0 gives no block key
 *   kv            num_planes == 2, num_kv_heads == 1, head_dim * element size a power
 *                 of two in [16, 1024] bytes; kv->cache_lengths is part of the cache's
 *                 description and not read by this operation
 *   ratio >= 1, 0 <= rotary_dim <= head_dim (even), eps >= 0 (the pages' string eps)
 * Launch bound: when kv->max_cache_length (host) is non-zero, blocks past
 * (kv->max_cache_length + max_prompt_length) / ratio are not computed, so key_counts
 * must not exceed that sum (a max_cache_length of 0 gives no such bound);
 * freqs_cis must hold every position a computed block starts at (checked on the host).
 * A block whose positions or pages do not address the cache is not written.
 * No workspace; asynchronous on `stream`.
 */
qsa_status qsa_compress_keys(void *block_keys, int64_t max_blocks, const void *gamma, const void *freqs_cis,
                             int32_t freq_dtype, int64_t num_positions, int64_t rotary_dim,
                             const int32_t *key_counts, const qsa_paged_cache *kv, int64_t batch,
                             uint32_t layer_idx, uint32_t max_prompt_length, int64_t ratio, float eps,
                             void *stream);

/* ------------------------------------------------------------------------- */
/* Block selection: the step between key compression and sparse attention. The
 * "QSACompressKeysPaged" page names its consumer (a block scorer that re-derives the
 * per-sequence stride max_blocks) but gives it no contract; the rule here is this
 * library's reading.
 *
 * Row r of sequence b, at position pos = cache_lengths[b] + (r - input_row_offsets[b]),
 * has nfull = (pos + 1) / ratio complete blocks and chooses among j < nv =
 * min(nfull, max_blocks). Block j scores q_index[r, :] . block_keys[b * max_blocks + j, :]
 * (fp32 sum of products). The k = min(topk, nv) highest scores are kept; equal scores go
 * to the lower block index. Output:
 *   token_indices[r, :]  the positions j*ratio .. j*ratio + ratio - 1 of the kept blocks in
 *                        increasing j, then the row's incomplete group nfull*ratio .. pos;
 *                        entries at or past counts[r] are not written
 *   counts[r]            k * ratio + (pos + 1 - nfull * ratio)
 *   blocks[r, 0:topk]    (optional, may be NULL) the kept j in increasing order, then -1
 * token_indices and counts are in the format qsa_sparse_attention reads.
 *
 *   q_index       ragged rows with num_q_heads == 1 (one index query per row), dtype F32 or
 *                 BF16, head_dim * element size a power of two in [16, 1024] bytes
 *   block_keys    [batch * max_blocks, head_dim] of q_index->dtype, 16-byte aligned (e.g.
 *                 qsa_compress_keys' block_keys); rows past a sequence's complete blocks
 *                 are never read
 *   cache_lengths [batch] (device); when max_cache_length (host) is non-zero, it and
 *                 q_index->max_prompt_length bound the candidates a launch covers:
 *                 min(max_blocks, their sum / ratio) must be at most 32768; with
 *                 max_cache_length 0, max_blocks itself must be
 *   selection_width >= topk * ratio + ratio - 1
 *   workspace     qsa_select_blocks_workspace_size bytes (fp32 scores), 16-byte aligned
 * Scores are fp32: blocks whose scores differ by less than fp32 rounding may be chosen
 * either way. The timing hook brackets both kernels of a call.
 */
qsa_status qsa_select_blocks_workspace_size(const qsa_ragged_q *q_index, int64_t max_blocks, int64_t ratio,
                                            int64_t topk, uint32_t max_cache_length, size_t *bytes);

qsa_status qsa_select_blocks(int32_t *token_indices, int64_t selection_width, int32_t *counts, int32_t *blocks,
                             const qsa_ragged_q *q_index, const void *block_keys, int64_t max_blocks,
                             const uint32_t *cache_lengths, uint32_t max_cache_length, int64_t ratio, int64_t topk,
                             void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------- */
/* Measurement aid, not one of the operations above: a plain streaming read of `bytes`
 * bytes at `src` (device, 16-byte aligned, bytes a multiple of 16), every byte loaded
 * once with 16-byte loads by `grid` workgroups of 256 threads; workgroup i writes one
 * word to sink[i] (device, `grid` words) so that the loads are kept. It is the
 * reference against which the gather kernels' bandwidth is read on the same GPU, and
 * a kernel of known traffic for scaling hardware byte counters. Asynchronous on
 * `stream`; 1 <= grid <= 2^20. */
qsa_status qsa_stream_read(const void *src, size_t bytes, uint32_t *sink, uint32_t grid, void *stream);

/* Measurement aid, not one of the operations above: a bare replay of a recorded
 * gather. Workgroup i < items (256 threads) reads, for every j < counts[i] (clamped to
 * [0, max_keys]), the row_bytes bytes at base + offsets[i * max_keys + j] and the
 * row_bytes bytes plane_delta further on (the K and V rows of a key), with 16-byte
 * non-temporal loads laid out as in the decode gather kernel (row_bytes / 16 lanes per
 * row, two batches of rows in flight per wavefront). A row whose bytes, in either plane, would fall outside
 * [base, base + region_bytes) is skipped. Thread t of workgroup i writes a fold of its
 * loads to sink[i * 256 + t] (device, items * 256 words). offsets (items * max_keys
 * int64, byte offsets) and counts (items int32) are device arrays; base is device
 * memory, 16-byte aligned, as is every offset. It gives the rate the access pattern
 * itself reaches on this GPU, without address computation or arithmetic.
 * row_bytes in {64, 128, 256, 512, 1024}; 1 <= max_keys <= 2^20; items <= 2^31 - 1;
 * region_bytes >= row_bytes when items > 0 (skipped keys load the region's first row
 * and do not fold it). Asynchronous on `stream`. */
qsa_status qsa_gather_replay(const void *base, uint64_t region_bytes, const int64_t *offsets, const int32_t *counts,
                             uint32_t items, uint32_t max_keys, uint32_t row_bytes, int64_t plane_delta,
                             uint32_t *sink, void *stream);

/* ------------------------------------------------------------------------- */
/* Text describing the last non-OK status returned on the calling thread. */
const char *qsa_last_error(void);

/* QSA_ABI_VERSION of the built library. */
int32_t qsa_abi_version(void);

/* sizeof() of the ABI structs as built: 0 = qsa_paged_cache, 1 = qsa_ragged_q,
 * 2 = qsa_launch_options; 0 for any other value. Lets bindings check their layout. */
size_t qsa_struct_size(int32_t which);

/* Profiling hook for the calling thread: when both are non-NULL, each later call on
 * this thread records `start` (a hipEvent_t) on its stream right before its main
 * gather kernel and `stop` right after it, so the caller can time that kernel alone.
 * Pass NULLs to stop. */
void qsa_set_timing_events(void *start, void *stop);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
