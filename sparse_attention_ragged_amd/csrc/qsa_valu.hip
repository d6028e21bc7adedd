// Dispatch of the wavefront gather kernel (groups of 1, 2 or 4 query heads per kv
// head) to its per-element-type instances.
#include "qsa_host.hpp"

#include <hip/hip_runtime.h>

namespace qsa {

int launch_gather_valu_f32(const GatherParams &p, void *stream);
int launch_gather_valu_bf16(const GatherParams &p, void *stream);
int launch_gather_valu_e4m3(const GatherParams &p, void *stream);

int launch_gather_valu(const GatherParams &p, void *stream)
{
    switch (p.dtype) {
    case QSA_F32: return launch_gather_valu_f32(p, stream);
    case QSA_BF16: return launch_gather_valu_bf16(p, stream);
    case QSA_FP8_E4M3: return launch_gather_valu_e4m3(p, stream);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace qsa
