// Wavefront gather kernel instances for bf16 keys and queries (every head_dim, group
// and key-list kind the wavefront path supports).
#include "qsa_valu_kernel.hpp"

namespace qsa {

int launch_gather_valu_bf16(const GatherParams &p, void *stream) { return launch_valu_lists<QSA_BF16>(p, stream); }

}  // namespace qsa
