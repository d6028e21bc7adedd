// Internal host-side interface of the library: launch parameter blocks, the
// validation/planning functions (pure C++, no HIP headers) and the kernel
// launchers implemented in the .hip translation units.
#pragma once

#include <cstddef>
#include <cstdint>

#include "qsa.h"

namespace qsa {

// Thread-local error text behind qsa_last_error().
qsa_status fail(qsa_status code, const char *fmt, ...);
void clear_error();

// Addressing of one paged cache leaf, in elements. The element offset of
// (page, plane, layer, slot, kv head, d) is
//   page * page_stride + plane * plane_stride + layer_off + slot * slot_stride + head * D + d.
//
// The kernels address in bytes with 32-bit in-page offsets (a page is smaller than
// 4 GiB, checked on the host): row = blocks + page * page_stride_b + (layer_off_b +
// slot * slot_stride_b + head_b), one 32x32->64 multiply-add per row.
struct CacheAddr {
    const void *blocks;
    const uint32_t *lut;
    int64_t page_stride;
    int64_t plane_stride;   // num_layers * page_size * Hkv * D
    int64_t layer_off;      // layer * page_size * Hkv * D
    int64_t slot_stride;    // Hkv * D
    int64_t max_pages;
    int64_t num_pages;
    int32_t page_size;
    int32_t magic_shift;    // position -> logical page: (pos * magic) >> magic_shift, exact for pos < 2^31
    uint64_t magic;
    int32_t page_shift;     // log2(page_size) when it is a power of two, else -1
    uint32_t page_mask;     // page_size - 1 (power of two)
    uint32_t page_stride_b; // the strides and the layer offset in bytes
    uint32_t plane_stride_b;
    uint32_t layer_off_b;
    uint32_t slot_stride_b;
};

// Key-list kinds the gather kernels walk for one (row, kv head).
enum KeyList : int32_t {
    KEYS_TOKEN_INDICES = 0,  // token_indices[r, 0:min(counts[r], W)]
    KEYS_BLOCKS = 1,         // block ids d_indices[g, r, 0:topk], block_size keys each, clipped at pos
    KEYS_LATENT = 2,         // window positions then comp_indices[r, :] >= 0
    KEYS_DENSE = 3,          // keys lo..hi of the row's own sequence in ragged k/v (no cache, no list)
};

struct GatherParams {
    void *out;
    int32_t out_dtype;
    int32_t dtype;
    const void *q;
    int64_t total_q;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t group;
    int32_t batch;
    int32_t layer;
    const uint32_t *row_off;
    const uint32_t *cache_lengths;   // positions (block-sparse, latent)
    CacheAddr kv;                    // K/V leaf, or the window leaf for latent
    CacheAddr comp;                  // compressed leaf (latent only)
    int32_t list_kind;
    int32_t block_size;
    int32_t block_shift;             // log2(block_size) when it is a power of two, else -1
    const int32_t *indices;          // token_indices / d_indices / comp_indices
    const int32_t *counts;           // token-index counts (KEYS_TOKEN_INDICES)
    int64_t width;                   // W, topk or num_comp
    int64_t window;                  // latent window
    const float *sink;               // latent sink logits or NULL
    const void *dense_k;             // dense: k, v [total_q, num_kv_heads, head_dim]
    const void *dense_v;
    int32_t dense_causal;            // dense: causal mask (the window is `window`, <= 0: none)
    float scale_log2;                // scale * log2(e)
    int32_t num_splits;
    int32_t waves;
    int32_t unroll;
    int64_t split_keys;              // keys per split (in key-list units)
    int64_t split_row0;              // rows before it run unsplit (head-split kernel's tail plan)
    int32_t head_block;              // wavefront kernel: kv heads one workgroup covers
    int32_t stream_rows;             // wavefront kernel: K/V row loads non-temporal (rows read once)
    float *ws_acc;                   // [S, total_q, Hq, D] when num_splits > 1
    float *ws_ml;                    // [S, total_q, Hq, 2]
};

enum GatherPath : int32_t {
    PATH_VALU = 0,        // groups of 1, 2, 4: wavefront dot products
    PATH_MFMA = 1,        // groups of 8..16: matrix cores, wavefronts split the keys
    PATH_MFMA_WIDE = 2,   // latent groups of 17..64: matrix cores, wavefronts split the heads
};

struct Plan {
    int32_t path;
    int32_t num_splits;
    int32_t waves;
    int32_t unroll;
    int64_t key_capacity;   // upper bound of keys per (row, kv head)
    int64_t split_keys;
    int64_t split_row0;     // rows before it run unsplit; the rest num_splits ways (0: all rows)
    int32_t head_block;     // wavefront kernel: kv heads per workgroup (1 for other paths)
    int32_t stream_rows;    // wavefront kernel: K/V row loads non-temporal
    size_t ws_bytes;
    size_t ws_ml_offset;
};

// Team layout of the wavefront kernel, shared by the kernel and the planner: a key's
// K (or V) row of one kv head is split over a team of lanes, each holding one or two
// 16-byte chunks (two where a lane then holds at most 16 elements).
constexpr int valu_chunks_per_lane(int elem_bytes, int head_dim)
{
    return head_dim * elem_bytes >= 64 && 2 * (16 / elem_bytes) <= 16 ? 2 : 1;
}
constexpr int valu_team_lanes(int elem_bytes, int head_dim)
{
    return head_dim * elem_bytes / (16 * valu_chunks_per_lane(elem_bytes, head_dim));
}

// Validation + planning (qsa_plan.cpp). They never touch the device.
qsa_status check_cache(const qsa_paged_cache *c, const char *what, int64_t planes);
qsa_status check_q(const qsa_ragged_q *q, const qsa_paged_cache *c, bool same_heads_as_cache);
qsa_status plan_gather(const qsa_ragged_q *q, int64_t num_kv_heads, int32_t dtype, int32_t list_kind,
                       int64_t key_capacity, int64_t split_unit, const qsa_launch_options *opts,
                       Plan *plan);
CacheAddr cache_addr(const qsa_paged_cache *c, uint32_t layer);

// Size of the library-owned device scratch behind qsa_sparse_attention_no_alloc
// (one copy per GPU, held until the process ends).
constexpr size_t kNoAllocScratchBytes = QSA_NO_ALLOC_SCRATCH_BYTES;

// Device address of the current device's scratch array (looked up once per device).
// Returns a hipError_t value (0 = success).
int scratch_address(void **ptr);

// Launchers (qsa_*.hip). Return a hipError_t value (0 = success).
int launch_gather_valu(const GatherParams &p, void *stream);
int launch_gather_mfma(const GatherParams &p, void *stream);
int launch_gather_mfma_wide(const GatherParams &p, void *stream);
int launch_splitk_combine(const GatherParams &p, void *stream);
int launch_stream_read(const void *src, uint64_t bytes, void *sink, uint32_t grid, void *stream);
int launch_gather_replay(const void *base, uint64_t region, const int64_t *offsets, const int32_t *counts,
                         uint32_t items, uint32_t max_keys, uint32_t row_bytes, int64_t plane_delta, uint32_t *sink,
                         void *stream);
int record_event(void *event, void *stream);
const char *hip_error_text(int err);

// Largest group of the head-split matrix-core kernel (16 heads per wavefront, four
// score wavefronts).
constexpr int kWideMaxGroup = 64;

// Which (dtype, group, head_dim) combinations have a built kernel (qsa_support.cpp).
bool valu_supported(int32_t dtype, int32_t group, int32_t head_dim);
bool mfma_supported(int32_t dtype, int32_t group, int32_t head_dim);
bool mfma_wide_supported(int32_t dtype, int32_t group, int32_t head_dim, int32_t list_kind);

}  // namespace qsa
