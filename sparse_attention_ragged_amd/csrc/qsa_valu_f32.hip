// Wavefront gather kernel instances for fp32 keys and queries (every head_dim, group
// and key-list kind the wavefront path supports).
#include "qsa_valu_kernel.hpp"

namespace qsa {

int launch_gather_valu_f32(const GatherParams &p, void *stream) { return launch_valu_lists<QSA_F32>(p, stream); }

}  // namespace qsa
