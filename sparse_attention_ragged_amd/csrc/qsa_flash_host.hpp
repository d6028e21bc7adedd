// Host-side interface of the dense ragged attention kernel with shared key tiles
// (qsa_mfma_flash.hip), kept apart from the gather kernels' interface in qsa_host.hpp.
#pragma once

#include "qsa_host.hpp"

namespace qsa {

// bf16, 8 to 16 query heads per kv head, head_dim 64, 128 or 256, one split.
bool mfma_flash_supported(int32_t dtype, int32_t group, int32_t head_dim);
int launch_gather_mfma_flash(const GatherParams &p, void *stream);

}  // namespace qsa
