/*
 * fp64 CPU oracle for index-selected sparse attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library may call, link or
 * include this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code with the HIP path.
 *
 * Every function evaluates the plain definition of the operation: exact softmax
 * attention over an explicitly listed key set, in double precision, on the
 * stored values decoded exactly to double. There is no blocking, no online
 * softmax and no reordering: per (row, head) it gathers the listed keys, forms
 * all scores, takes their maximum, exponentiates, and divides. OpenMP only runs
 * independent output rows at the same time.
 *
 * Sources (Modular MAX API pages):
 *   - "QSASparseAttentionRaggedPaged": Tensor shapes list, execute() Args
 *     (kv_blocks [num_pages, 2, num_layers, page_size, num_kv_heads, head_dim],
 *     kv_lookup_table [batch, max_pages], token_indices [total_q, selection_width],
 *     counts [total_q]; entries at or past counts are never read; group = query
 *     heads per kv head; page_stride = page-to-page distance, -1 when packed).
 *   - "Struct_msa_attention_ragged_paged": design notes and Args (topk block ids
 *     per (kv head, query token) in d_indices [n_kv_heads, num_rows, topk];
 *     e4m3 is scale-free; FP32 accumulation; output always BF16).
 *   - "latent_sparse_attention_ragged_paged": summary, Parameters and Args
 *     (window keys max(0, pos-window+1)..pos, listed compressed entries with -1
 *     marking an unused slot, per-head sink logits, scale applied to scores).
 *
 *   - "RaggedFlashAttentionGPU": summary, Parameters and Args (ragged q, k, v
 *     [total_seq_len, heads, head_dim] without a KV cache, input_row_offsets,
 *     a mask type and an optional local window size, -1 for none).
 *   - "QSACompressKeysPaged": summary, Tensor shapes, execute Parameters and Args
 *     (block_keys [batch * max_blocks, head_dim], gamma [head_dim], freqs_cis
 *     [positions, rotary_dim] of cos/sin pairs, key_counts = raw keys per sequence
 *     this step included, ratio, rotary_dim, eps; the per-sequence stride max_blocks
 *     that the block scorer re-derives, which names the selection step).
 *
 * Readings where the pages are silent (listed in the design notes of the repo):
 *   - query head h reads kv head h / group (consecutive groups);
 *   - a row's position is cache_lengths[b] + (row - input_row_offsets[b]);
 *   - counts <= 0 gives an all-zero output row; counts > selection_width is
 *     clamped to selection_width; duplicated indices count with multiplicity;
 *   - latent leaves hold one plane: the same latent row is key and value;
 *   - the sink logit is not multiplied by scale and carries a zero value row;
 *   - dense ragged attention: row i of a sequence (0-based within it) sees the
 *     keys j of its own sequence with j <= i under the causal mask (all j of the
 *     sequence without a mask) and, with a local window w > 0, j >= i - w + 1;
 *     k and v may have fewer heads than q (query head h reads kv head h / group);
 *   - key compression (parity unpinned for these choices: no page value fixes them):
 *     the pooling is the mean of a complete group of `ratio` consecutive raw keys (a
 *     trailing partial group gives no block key); the order is pool, then RMS-norm
 *     with gamma, then rotation; the rotation turns interleaved channel pairs
 *     (2i, 2i+1) below rotary_dim by the table's (cos, sin) pair at the block's first
 *     raw position j * ratio; raw keys sit in plane 0 (K) of the indexer cache;
 *   - block selection (no page gives its contract; parity unpinned for these choices):
 *     one index query vector per row, the score of a block is its dot product with the
 *     block key, the top-k complete blocks are kept (equal scores: lower index first),
 *     the row always keeps its incomplete group, and positions are emitted in
 *     increasing order.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * (closed forms, invariants, brute-force dense masked attention, exhaustive
 * codec checks); see that file for which pin covers which step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2 };
enum { ORC_OK = 0, ORC_EINPUT = 1, ORC_ENOMEM = 2 };

/* ----------------------------------------------------------------- decoders */

/* bf16 is the upper half of an IEEE-754 binary32: widen by placing the 16 bits
 * on top of 16 zero bits and reading the result as binary32. */
static double dec_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit E4M3 ("fn" variant): 1 sign bit, 4 exponent bits (bias 7),
 * 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
 * there is no infinity. */
static double dec_e4m3(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

static double elem(const void *base, int dt, int64_t i)
{
    switch (dt) {
    case ORC_F32: return (double)((const float *)base)[i];
    case ORC_BF16: return dec_bf16(((const uint16_t *)base)[i]);
    default: return dec_e4m3(((const uint8_t *)base)[i]);
    }
}

int orc_decode(int dt, const void *src, double *dst, int64_t n)
{
    if (dt < ORC_F32 || dt > ORC_E4M3)
        return ORC_EINPUT;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = elem(src, dt, i);
    return ORC_OK;
}

/* ------------------------------------------------------------ paged caches */

typedef struct {
    const void *blocks;
    int dt;
    int64_t num_pages, planes, num_layers, page_size, num_kv_heads, head_dim;
    int64_t page_stride; /* elements between pages; -1 = packed */
    const uint32_t *lut;
    int64_t max_pages;
    const uint32_t *cache_lengths;
} orc_cache;

/* Decode row (plane, layer, position p of sequence b, kv head g) into dst[head_dim].
 * The page of position p is lut[b, p / page_size] and its slot p % page_size;
 * inside a page the layout is packed [planes, num_layers, page_size, Hkv, D]. */
static int gather_row(const orc_cache *c, int64_t b, int64_t p, int64_t plane, int64_t layer,
                      int64_t g, double *dst)
{
    if (p < 0 || p >= c->page_size * c->max_pages)
        return ORC_EINPUT;
    int64_t page = c->lut[b * c->max_pages + p / c->page_size];
    int64_t slot = p % c->page_size;
    if (page >= c->num_pages)
        return ORC_EINPUT;
    int64_t packed = c->planes * c->num_layers * c->page_size * c->num_kv_heads * c->head_dim;
    int64_t stride = c->page_stride == -1 ? packed : c->page_stride;
    int64_t off = page * stride +
                  (((plane * c->num_layers + layer) * c->page_size + slot) * c->num_kv_heads + g) *
                      c->head_dim;
    for (int64_t d = 0; d < c->head_dim; ++d)
        dst[d] = elem(c->blocks, c->dt, off + d);
    return ORC_OK;
}

static int64_t seq_of_row(const uint32_t *row_off, int64_t batch, int64_t r)
{
    for (int64_t b = 0; b < batch; ++b)
        if ((int64_t)row_off[b] <= r && r < (int64_t)row_off[b + 1])
            return b;
    return -1;
}

/* Softmax attention of one query vector over n listed key rows.
 *   s_j = scale * sum_d q[d] K[j][d]
 *   out = sum_j exp(s_j - m) V[j] / (sum_j exp(s_j - m) + exp(sink - m)),
 *   m = max(max_j s_j, sink)
 * A sink of -INFINITY contributes nothing (plain softmax). With no keys and no
 * finite sink the output is zero. */
static void attend(const double *qv, const double *K, const double *V, int64_t n, int64_t D,
                   double scale, double sink, double *s, double *out)
{
    for (int64_t d = 0; d < D; ++d)
        out[d] = 0.0;
    if (n <= 0)
        return;
    double m = sink;
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += qv[d] * K[j * D + d];
        s[j] = scale * acc;
        if (s[j] > m)
            m = s[j];
    }
    double z = exp(sink - m); /* 0 for a sink of -INFINITY */
    for (int64_t j = 0; j < n; ++j) {
        double w = exp(s[j] - m);
        z += w;
        for (int64_t d = 0; d < D; ++d)
            out[d] += w * V[j * D + d];
    }
    for (int64_t d = 0; d < D; ++d)
        out[d] /= z;
}

static int check_rows(const int64_t *rows, int64_t n_rows, int64_t total_q)
{
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t r = rows ? rows[i] : i;
        if (r < 0 || r >= total_q)
            return ORC_EINPUT;
    }
    return ORC_OK;
}

/* -------------------------------------------------------------------- QSA */

/* Index-selected sparse GQA ("QSASparseAttentionRaggedPaged").
 * out[i, h, :] for query row r = rows[i] (or i when rows is NULL):
 *   n = min(counts[r], W); keys j < n at positions token_indices[r, j] of r's
 *   sequence, kv head h / group, layer layer_idx; softmax(scale * q.K) . V. */
int orc_qsa(double *out, const int64_t *rows, int64_t n_rows,
            const void *q, int dt, int64_t total_q, int64_t Hq, int64_t D,
            const uint32_t *row_off, int64_t batch,
            const void *kv, int64_t num_pages, int64_t num_layers, int64_t page_size,
            int64_t Hkv, int64_t page_stride, const uint32_t *cache_lengths,
            const uint32_t *lut, int64_t max_pages, int64_t layer_idx,
            const int32_t *token_indices, int64_t W, const int32_t *counts, float scale,
            int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv || layer_idx < 0 || layer_idx >= num_layers ||
        check_rows(rows, n_rows, total_q))
        return ORC_EINPUT;
    orc_cache c = {kv, dt, num_pages, 2, num_layers, page_size, Hkv, D, page_stride,
                   lut, max_pages, cache_lengths};
    int64_t G = Hq / Hkv;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *K = malloc(sizeof(double) * (W > 0 ? W : 1) * D);
        double *V = malloc(sizeof(double) * (W > 0 ? W : 1) * D);
        double *s = malloc(sizeof(double) * (W > 0 ? W : 1));
        double *qv = malloc(sizeof(double) * D);
        if (!K || !V || !s || !qv) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (err)
                continue;
            int64_t r = rows ? rows[i] : i;
            int64_t b = seq_of_row(row_off, batch, r);
            int64_t n = counts[r] < W ? counts[r] : W;
            double *o = out + i * Hq * D;
            if (b < 0) {
#pragma omp atomic write
                err = ORC_EINPUT;
                continue;
            }
            for (int64_t g = 0; g < Hkv; ++g) {
                int bad = 0;
                for (int64_t j = 0; j < n && !bad; ++j) {
                    int64_t p = token_indices[r * W + j];
                    bad |= gather_row(&c, b, p, 0, layer_idx, g, K + j * D);
                    bad |= gather_row(&c, b, p, 1, layer_idx, g, V + j * D);
                }
                if (bad) {
#pragma omp atomic write
                    err = ORC_EINPUT;
                    break;
                }
                for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                    for (int64_t d = 0; d < D; ++d)
                        qv[d] = elem(q, dt, (r * Hq + h) * D + d);
                    attend(qv, K, V, n, D, (double)scale, -INFINITY, s, o + h * D);
                }
            }
        }
        free(K);
        free(V);
        free(s);
        free(qv);
    }
    return err;
}

/* ----------------------------------------------------------- block-sparse */

/* Block-sparse top-k attention ("Struct_msa_attention_ragged_paged").
 * For row r at position pos and kv head g the keys are, for each listed block
 * id t in d_indices[g, r, :], the positions block_size*t + i (0 <= i < block_size)
 * that are <= pos. Every q head of group g attends to them. */
int orc_block_sparse(double *out, const int64_t *rows, int64_t n_rows,
                     const void *q, int dt, int64_t total_q, int64_t Hq, int64_t D,
                     const uint32_t *row_off, int64_t batch,
                     const void *kv, int64_t num_pages, int64_t num_layers, int64_t page_size,
                     int64_t Hkv, int64_t page_stride, const uint32_t *cache_lengths,
                     const uint32_t *lut, int64_t max_pages, int64_t layer_idx,
                     const int32_t *d_indices, int64_t topk, int64_t block_size, float scale,
                     int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv || layer_idx < 0 || layer_idx >= num_layers || block_size <= 0 ||
        topk < 0 || check_rows(rows, n_rows, total_q))
        return ORC_EINPUT;
    orc_cache c = {kv, dt, num_pages, 2, num_layers, page_size, Hkv, D, page_stride,
                   lut, max_pages, cache_lengths};
    int64_t G = Hq / Hkv;
    int64_t cap = (topk > 0 ? topk : 1) * block_size;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *K = malloc(sizeof(double) * cap * D);
        double *V = malloc(sizeof(double) * cap * D);
        double *s = malloc(sizeof(double) * cap);
        double *qv = malloc(sizeof(double) * D);
        if (!K || !V || !s || !qv) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (err)
                continue;
            int64_t r = rows ? rows[i] : i;
            int64_t b = seq_of_row(row_off, batch, r);
            if (b < 0) {
#pragma omp atomic write
                err = ORC_EINPUT;
                continue;
            }
            int64_t pos = (int64_t)cache_lengths[b] + (r - (int64_t)row_off[b]);
            double *o = out + i * Hq * D;
            for (int64_t g = 0; g < Hkv; ++g) {
                int64_t n = 0;
                int bad = 0;
                for (int64_t t = 0; t < topk && !bad; ++t) {
                    int64_t id = d_indices[(g * total_q + r) * topk + t];
                    if (id < 0) {
                        bad = 1;
                        break;
                    }
                    for (int64_t k = 0; k < block_size; ++k) {
                        int64_t p = id * block_size + k;
                        if (p > pos)
                            break;
                        bad |= gather_row(&c, b, p, 0, layer_idx, g, K + n * D);
                        bad |= gather_row(&c, b, p, 1, layer_idx, g, V + n * D);
                        ++n;
                    }
                }
                if (bad) {
#pragma omp atomic write
                    err = ORC_EINPUT;
                    break;
                }
                for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                    for (int64_t d = 0; d < D; ++d)
                        qv[d] = elem(q, dt, (r * Hq + h) * D + d);
                    attend(qv, K, V, n, D, (double)scale, -INFINITY, s, o + h * D);
                }
            }
        }
        free(K);
        free(V);
        free(s);
        free(qv);
    }
    return err;
}

/* ----------------------------------------------------------------- latent */

/* Latent window + compressed + sink attention ("latent_sparse_attention_ragged_paged").
 * Row r at position pos (from the window leaf's cache_lengths) attends to
 *   X = [window rows at positions max(0, pos-window+1) .. pos]
 *       ++ [compressed rows at entries e = comp_indices[r, t] for which e >= 0];
 * each x is one latent row (key and value at once), and head h adds the sink
 * logit attn_sink[h] (unscaled, zero value) to the softmax denominator. */
int orc_latent(double *out, const int64_t *rows, int64_t n_rows,
               const void *q, int dt, int64_t total_q, int64_t Hq, int64_t D,
               const uint32_t *row_off, int64_t batch,
               const void *swa, int64_t swa_pages, int64_t swa_layers, int64_t swa_ps,
               int64_t swa_stride, const uint32_t *swa_cache_lengths, const uint32_t *swa_lut,
               int64_t swa_max_pages,
               const void *comp, int64_t comp_pages, int64_t comp_layers, int64_t comp_ps,
               int64_t comp_stride, const uint32_t *comp_lut, int64_t comp_max_pages,
               int64_t layer_idx, int64_t window, const int32_t *comp_indices, int64_t num_comp,
               const float *attn_sink, float scale, int nthreads)
{
    if (window <= 0 || num_comp < 0 || layer_idx < 0 || layer_idx >= swa_layers ||
        layer_idx >= comp_layers || check_rows(rows, n_rows, total_q))
        return ORC_EINPUT;
    orc_cache cs = {swa, dt, swa_pages, 1, swa_layers, swa_ps, 1, D, swa_stride,
                    swa_lut, swa_max_pages, swa_cache_lengths};
    orc_cache cc = {comp, dt, comp_pages, 1, comp_layers, comp_ps, 1, D, comp_stride,
                    comp_lut, comp_max_pages, NULL};
    int64_t cap = window + num_comp;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *X = malloc(sizeof(double) * (cap > 0 ? cap : 1) * D);
        double *s = malloc(sizeof(double) * (cap > 0 ? cap : 1));
        double *qv = malloc(sizeof(double) * D);
        if (!X || !s || !qv) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (err)
                continue;
            int64_t r = rows ? rows[i] : i;
            int64_t b = seq_of_row(row_off, batch, r);
            if (b < 0) {
#pragma omp atomic write
                err = ORC_EINPUT;
                continue;
            }
            int64_t pos = (int64_t)swa_cache_lengths[b] + (r - (int64_t)row_off[b]);
            int64_t lo = pos - window + 1 > 0 ? pos - window + 1 : 0;
            int64_t n = 0;
            int bad = 0;
            for (int64_t p = lo; p <= pos && !bad; ++p)
                bad |= gather_row(&cs, b, p, 0, layer_idx, 0, X + (n++) * D);
            for (int64_t t = 0; t < num_comp && !bad; ++t) {
                int64_t e = comp_indices[r * num_comp + t];
                if (e >= 0)
                    bad |= gather_row(&cc, b, e, 0, layer_idx, 0, X + (n++) * D);
            }
            if (bad) {
#pragma omp atomic write
                err = ORC_EINPUT;
                continue;
            }
            double *o = out + i * Hq * D;
            for (int64_t h = 0; h < Hq; ++h) {
                for (int64_t d = 0; d < D; ++d)
                    qv[d] = elem(q, dt, (r * Hq + h) * D + d);
                attend(qv, X, X, n, D, (double)scale, (double)attn_sink[h], s, o + h * D);
            }
        }
        free(X);
        free(s);
        free(qv);
    }
    return err;
}

/* ------------------------------------------------------------ dense ragged */

/* Dense ragged attention without a KV cache ("RaggedFlashAttentionGPU").
 * For query row r of sequence b, i = r - row_off[b], L = row_off[b+1] - row_off[b]:
 *   keys j in [lo, hi], hi = causal ? i : L - 1, lo = window > 0 ? max(0, i - window + 1) : 0,
 *   K_j = k[row_off[b] + j, h / group, :], V_j likewise; softmax(scale * q.K) . V. */
int orc_dense(double *out, const int64_t *rows, int64_t n_rows,
              const void *q, const void *k, const void *v, int dt, int64_t total_q, int64_t Hq,
              int64_t Hkv, int64_t D, const uint32_t *row_off, int64_t batch, int causal,
              int64_t window, float scale, int nthreads)
{
    if (Hkv <= 0 || Hq % Hkv || check_rows(rows, n_rows, total_q))
        return ORC_EINPUT;
    int64_t G = Hq / Hkv;
    int64_t maxlen = 1;
    for (int64_t b = 0; b < batch; ++b)
        if ((int64_t)row_off[b + 1] - (int64_t)row_off[b] > maxlen)
            maxlen = (int64_t)row_off[b + 1] - (int64_t)row_off[b];
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *K = malloc(sizeof(double) * maxlen * D);
        double *V = malloc(sizeof(double) * maxlen * D);
        double *s = malloc(sizeof(double) * maxlen);
        double *qv = malloc(sizeof(double) * D);
        if (!K || !V || !s || !qv) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (err)
                continue;
            int64_t r = rows ? rows[i] : i;
            int64_t b = seq_of_row(row_off, batch, r);
            if (b < 0) {
#pragma omp atomic write
                err = ORC_EINPUT;
                continue;
            }
            int64_t start = row_off[b], len = (int64_t)row_off[b + 1] - start, t = r - start;
            int64_t hi = causal ? t : len - 1;
            int64_t lo = window > 0 && t - window + 1 > 0 ? t - window + 1 : 0;
            int64_t n = hi - lo + 1;
            double *o = out + i * Hq * D;
            for (int64_t g = 0; g < Hkv; ++g) {
                for (int64_t j = 0; j < n; ++j)
                    for (int64_t d = 0; d < D; ++d) {
                        K[j * D + d] = elem(k, dt, ((start + lo + j) * Hkv + g) * D + d);
                        V[j * D + d] = elem(v, dt, ((start + lo + j) * Hkv + g) * D + d);
                    }
                for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                    for (int64_t d = 0; d < D; ++d)
                        qv[d] = elem(q, dt, (r * Hq + h) * D + d);
                    attend(qv, K, V, n, D, (double)scale, -INFINITY, s, o + h * D);
                }
            }
        }
        free(K);
        free(V);
        free(s);
        free(qv);
    }
    return err;
}

/* ---------------------------------------------------------- key compression */

/* Block keys pooled from raw index keys ("QSACompressKeysPaged": summary, Tensor
 * shapes, execute Parameters and Args). Sequence b holds key_counts[b] raw keys at
 * positions 0.. of plane 0, kv head 0 of the indexer cache; its complete groups of
 * `ratio` consecutive keys become n_b = min(key_counts[b] / ratio, max_blocks) block
 * keys, block j covering positions j*ratio .. j*ratio + ratio - 1. For block j:
 *   pooled_d = (1 / ratio) * sum_t K[j*ratio + t]_d                 (mean pool)
 *   normed_d = gamma_d * pooled_d / sqrt((1 / D) * sum_e pooled_e^2 + eps)
 *   with c = F[j*ratio][2i], s = F[j*ratio][2i + 1] for each channel pair with
 *   2i + 1 < rotary_dim, the pair turns by the angle whose cosine and sine those are:
 *   out_2i = c * normed_2i - s * normed_2i+1, out_2i+1 = s * normed_2i + c * normed_2i+1;
 *   channels at or past rotary_dim keep normed_d.
 * Output rows b * max_blocks + j for j >= n_b are not produced: they are NaN here. */
int orc_compress(double *out, const void *blocks, int dt, int64_t num_pages, int64_t planes,
                 int64_t num_layers, int64_t page_size, int64_t D, int64_t page_stride,
                 const uint32_t *lut, int64_t max_pages, int64_t layer_idx, const int32_t *key_counts,
                 int64_t batch, int64_t max_blocks, int64_t ratio, const void *gamma,
                 const void *freqs, int fdt, int64_t num_positions, int64_t rotary_dim, float eps,
                 int nthreads)
{
    if (ratio < 1 || max_blocks < 0 || rotary_dim < 0 || rotary_dim % 2 || rotary_dim > D ||
        layer_idx < 0 || layer_idx >= num_layers)
        return ORC_EINPUT;
    orc_cache c = {blocks, dt, num_pages, planes, num_layers, page_size, 1, D,
                   page_stride, lut, max_pages, NULL};
    for (int64_t i = 0; i < batch * max_blocks * D; ++i)
        out[i] = NAN;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        double *row = malloc(sizeof(double) * D);
        double *x = malloc(sizeof(double) * D);
        if (!row || !x) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for collapse(2) schedule(dynamic, 64)
        for (int64_t b = 0; b < batch; ++b)
            for (int64_t j = 0; j < max_blocks; ++j) {
                int64_t nb = key_counts[b] > 0 ? key_counts[b] / ratio : 0;
                if (err || j >= nb)
                    continue;
                for (int64_t d = 0; d < D; ++d)
                    x[d] = 0.0;
                int bad = 0;
                for (int64_t t = 0; t < ratio; ++t) {
                    bad |= gather_row(&c, b, j * ratio + t, 0, layer_idx, 0, row);
                    for (int64_t d = 0; d < D; ++d)
                        x[d] += row[d];
                }
                int64_t p = j * ratio;
                if (bad || (rotary_dim > 0 && p >= num_positions)) {
#pragma omp atomic write
                    err = ORC_EINPUT;
                    continue;
                }
                for (int64_t d = 0; d < D; ++d)
                    x[d] /= (double)ratio;
                double ss = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    ss += x[d] * x[d];
                double inv = 1.0 / sqrt(ss / (double)D + (double)eps);
                for (int64_t d = 0; d < D; ++d)
                    x[d] = elem(gamma, dt, d) * x[d] * inv;
                double *o = out + (b * max_blocks + j) * D;
                for (int64_t d = 0; d < D; ++d)
                    o[d] = x[d];
                for (int64_t i = 0; 2 * i + 1 < rotary_dim; ++i) {
                    double cs = elem(freqs, fdt, p * rotary_dim + 2 * i);
                    double sn = elem(freqs, fdt, p * rotary_dim + 2 * i + 1);
                    o[2 * i] = cs * x[2 * i] - sn * x[2 * i + 1];
                    o[2 * i + 1] = sn * x[2 * i] + cs * x[2 * i + 1];
                }
            }
        free(row);
        free(x);
    }
    return err;
}

/* ------------------------------------------------------- selection producer */

typedef struct {
    double s;
    int64_t j;
} orc_scored;

/* Higher score first; equal scores: lower block index first. */
static int cmp_scored(const void *a, const void *b)
{
    const orc_scored *x = a, *y = b;
    if (x->s != y->s)
        return x->s > y->s ? -1 : 1;
    return x->j < y->j ? -1 : x->j > y->j;
}

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return x < y ? -1 : x > y;
}

/* Block selection from block keys (the step "QSACompressKeysPaged" names as the
 * consumer of its block keys, qsa_block_score, followed by a top-k). Row r of sequence b
 * at position pos = cache_lengths[b] + (r - row_off[b]) has (pos + 1) / ratio complete
 * blocks and sees those with j < nv = min((pos + 1) / ratio, max_blocks); block j scores
 * s_j = sum_d q_index[r, d] * block_keys[b * max_blocks + j, d]. The k = min(topk, nv)
 * highest scores are kept (equal scores: the lower block index first). Output, per row:
 * token_indices[r, :] = the positions j*ratio .. j*ratio + ratio - 1 of the kept blocks
 * in increasing j, then the positions of the row's incomplete group,
 * ((pos + 1) / ratio) * ratio .. pos (fewer than ratio); counts[r] = k*ratio + that
 * group's size; blocks[r, 0:k] = the kept j in increasing
 * order and -1 after (when blocks is not NULL). Entries of token_indices at or past
 * counts[r] are left as they were. */
int orc_select(int32_t *token_indices, int32_t *counts, int32_t *blocks, const void *q_index,
               const void *block_keys, int dt, int64_t total_q, int64_t D, const uint32_t *row_off,
               const uint32_t *cache_lengths, int64_t batch, int64_t max_blocks, int64_t ratio, int64_t topk,
               int64_t W, int nthreads)
{
    if (ratio < 1 || topk < 0 || max_blocks < 0 || W < topk * ratio + ratio - 1)
        return ORC_EINPUT;
    int err = ORC_OK;
#pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1)
    {
        orc_scored *sc = malloc(sizeof(orc_scored) * (max_blocks > 0 ? max_blocks : 1));
        int64_t *kept = malloc(sizeof(int64_t) * (topk > 0 ? topk : 1));
        if (!sc || !kept) {
#pragma omp atomic write
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < total_q; ++r) {
            if (err)
                continue;
            int64_t b = seq_of_row(row_off, batch, r);
            if (b < 0) {
#pragma omp atomic write
                err = ORC_EINPUT;
                continue;
            }
            int64_t pos = (int64_t)cache_lengths[b] + (r - (int64_t)row_off[b]);
            int64_t nfull = (pos + 1) / ratio;
            int64_t nv = nfull < max_blocks ? nfull : max_blocks;
            for (int64_t j = 0; j < nv; ++j) {
                double s = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    s += elem(q_index, dt, r * D + d) * elem(block_keys, dt, (b * max_blocks + j) * D + d);
                sc[j].s = s;
                sc[j].j = j;
            }
            int64_t k = topk < nv ? topk : nv;
            qsort(sc, (size_t)nv, sizeof(orc_scored), cmp_scored);
            for (int64_t m = 0; m < k; ++m)
                kept[m] = sc[m].j;
            qsort(kept, (size_t)k, sizeof(int64_t), cmp_i64);
            int64_t n = 0;
            for (int64_t m = 0; m < k; ++m)
                for (int64_t t = 0; t < ratio; ++t)
                    token_indices[r * W + n++] = (int32_t)(kept[m] * ratio + t);
            for (int64_t p = nfull * ratio; p <= pos; ++p)
                token_indices[r * W + n++] = (int32_t)p;
            counts[r] = (int32_t)n;
            if (blocks)
                for (int64_t m = 0; m < topk; ++m)
                    blocks[r * topk + m] = m < k ? (int32_t)kept[m] : -1;
        }
        free(sc);
        free(kept);
    }
    return err;
}
