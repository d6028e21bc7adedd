// Host-only stand-ins for the library's device side, for building the C-ABI argument
// checks and launch planning (qsa_api.cpp, qsa_plan.cpp, qsa_support.cpp) without HIP,
// under address and undefined-behaviour sanitizers. A "launch" only counts itself and
// checks the sizes it was given; nothing is dereferenced.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "qsa_host.hpp"
#include "qsa_select_host.hpp"
#include "qsa_flash_host.hpp"

namespace qsa {

long g_launches = 0;

static void check_gather(const GatherParams &p)
{
    // every split-K plan must have brought a workspace
    if (p.num_splits > 1 && (!p.ws_acc || !p.ws_ml)) {
        std::fprintf(stderr, "split-K launch without partials\n");
        std::abort();
    }
    if (p.total_q <= 0 || p.num_splits < 1 || p.waves < 1) {
        std::fprintf(stderr, "launch of an empty or invalid plan\n");
        std::abort();
    }
    ++g_launches;
}

int launch_gather_valu(const GatherParams &p, void *) { check_gather(p); return 0; }
int launch_gather_mfma(const GatherParams &p, void *) { check_gather(p); return 0; }
int launch_gather_mfma_wide(const GatherParams &p, void *) { check_gather(p); return 0; }
int launch_gather_mfma_flash(const GatherParams &p, void *) { check_gather(p); return 0; }
int launch_splitk_combine(const GatherParams &p, void *) { check_gather(p); return 0; }
int launch_stream_read(const void *, uint64_t, void *, uint32_t, void *) { ++g_launches; return 0; }
int launch_gather_replay(const void *, uint64_t, const int64_t *, const int32_t *, uint32_t, uint32_t, uint32_t, int64_t,
                         uint32_t *, void *)
{
    ++g_launches;
    return 0;
}
int launch_compress_keys(const CompressParams &p, void *)
{
    if (p.batch < 1 || p.blocks_bound < 1)
        std::abort();
    ++g_launches;
    return 0;
}
int launch_select_blocks(const SelectParams &p, void *, void *, void *)
{
    if (p.total_q < 1)
        std::abort();
    ++g_launches;
    return 0;
}
int record_event(void *, void *) { return 0; }
const char *hip_error_text(int) { return "stub"; }

static unsigned char g_scratch[256];
int scratch_address(void **ptr)
{
    *ptr = g_scratch;
    return 0;
}

}  // namespace qsa
