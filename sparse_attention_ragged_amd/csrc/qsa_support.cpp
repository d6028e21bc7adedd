// Which (dtype, group, head_dim, list) combinations each kernel family is built for.
// Pure host logic, kept apart from the device translation units so that the argument
// checks can be built and tested without HIP (the launchers in the .hip files
// instantiate exactly these combinations).
#include "qsa_host.hpp"
#include "qsa_select_host.hpp"
#include "qsa_flash_host.hpp"

namespace qsa {

bool valu_supported(int32_t dtype, int32_t group, int32_t head_dim)
{
    return (dtype == QSA_F32 || dtype == QSA_BF16 || dtype == QSA_FP8_E4M3) &&
           (group == 1 || group == 2 || group == 4) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

bool mfma_supported(int32_t dtype, int32_t group, int32_t head_dim)
{
    return (dtype == QSA_BF16 || dtype == QSA_FP8_E4M3) && group >= 8 && group <= 16 &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

bool mfma_wide_supported(int32_t dtype, int32_t group, int32_t head_dim, int32_t list_kind)
{
    return dtype == QSA_BF16 && list_kind == KEYS_LATENT && group > 16 && group <= kWideMaxGroup &&
           (head_dim == 128 || head_dim == 256 || head_dim == 512);
}

bool mfma_flash_supported(int32_t dtype, int32_t group, int32_t head_dim)
{
    return dtype == QSA_BF16 && group >= 8 && group <= 16 && (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

bool compress_supported(int32_t dtype, int32_t head_dim)
{
    if (dtype != QSA_F32 && dtype != QSA_BF16)
        return false;
    const int64_t bytes = (int64_t)head_dim * (dtype == QSA_F32 ? 4 : 2);
    return bytes >= 16 && bytes <= 1024 && bytes % 16 == 0 && ((bytes / 16) & (bytes / 16 - 1)) == 0;
}

bool select_supported(int32_t dtype, int32_t head_dim)
{
    if (dtype != QSA_F32 && dtype != QSA_BF16)
        return false;
    const int64_t bytes = (int64_t)head_dim * (dtype == QSA_F32 ? 4 : 2);
    return bytes >= 16 && bytes <= 1024 && ((bytes / 16) & (bytes / 16 - 1)) == 0 && bytes % 16 == 0;
}

}  // namespace qsa
