// Wavefront gather kernel instances for OCP e4m3 keys and queries (every head_dim, group
// and key-list kind the wavefront path supports).
#include "qsa_valu_kernel.hpp"

namespace qsa {

int launch_gather_valu_e4m3(const GatherParams &p, void *stream) { return launch_valu_lists<QSA_FP8_E4M3>(p, stream); }

}  // namespace qsa
