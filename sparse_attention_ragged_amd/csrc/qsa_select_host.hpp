// Host-side interface of the two steps that produce a selection (key compression and
// block selection): parameter blocks and launchers, kept apart from the gather
// kernels' interface in qsa_host.hpp.
#pragma once

#include "qsa_host.hpp"

namespace qsa {

// Key compression: one team of lanes per block key (qsa_compress.hip).
struct CompressParams {
    void *out;                   // block_keys [batch * max_blocks, head_dim], element type `dtype`
    const void *gamma;           // [head_dim], element type `dtype`
    const void *freqs;           // [num_positions, rotary_dim] of freq_dtype (cos, sin pairs)
    const int32_t *key_counts;   // [batch]
    CacheAddr kv;                // plane 0 (raw keys), kv head 0, the addressed layer
    int64_t max_blocks;          // row stride of one sequence in `out`
    int64_t blocks_bound;        // blocks per sequence the grid covers (host-side bound)
    int32_t dtype;
    int32_t freq_dtype;
    int32_t head_dim;
    int32_t rotary_dim;
    int32_t ratio;
    int32_t batch;
    float eps;
};

// Threads of a compression workgroup, and the lanes that share one raw key row there
// (one 16-byte chunk each).
constexpr int kCompressThreads = 256;
constexpr int compress_team_lanes(int elem_bytes, int head_dim) { return head_dim * elem_bytes / 16; }

// Block selection (qsa_select.hip): scores of every visible block, then a top-k per row.
struct SelectParams {
    int32_t *token_indices;      // [total_q, width]
    int32_t *counts;             // [total_q]
    int32_t *blocks;             // [total_q, topk] or NULL
    const void *q_index;         // [total_q, head_dim], element type `dtype`
    const void *block_keys;      // [batch * max_blocks, head_dim], element type `dtype`
    const uint32_t *row_off;     // [batch + 1]
    const uint32_t *cache_lengths;
    float *scores;               // workspace [total_q, cand_bound]
    int64_t total_q;
    int64_t width;
    int64_t max_blocks;
    int64_t cand_bound;          // candidate blocks per row the launch covers
    int32_t batch;
    int32_t dtype;
    int32_t head_dim;
    int32_t ratio;
    int32_t topk;
};
constexpr int64_t kSelectMaxCandidates = 32768;   // one row's scores in LDS (128 KiB)

int launch_compress_keys(const CompressParams &p, void *stream);
int launch_select_blocks(const SelectParams &p, void *stream, void *ev_start, void *ev_stop);

// Which (dtype, head_dim) combinations have a built kernel.
bool compress_supported(int32_t dtype, int32_t head_dim);
bool select_supported(int32_t dtype, int32_t head_dim);

}  // namespace qsa
