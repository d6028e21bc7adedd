// Gather-attention on matrix cores (groups of 8 or more query heads per kv head).
#include "qsa_device.hpp"

namespace qsa {

bool mfma_supported(int32_t, int32_t, int32_t) { return false; }

int launch_gather_mfma(const GatherParams &, void *) { return (int)hipErrorInvalidValue; }

}  // namespace qsa
