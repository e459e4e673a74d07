// Attention kernels with 4 query heads per kv head (grouped-query
// attention): head dims 256 and 128, 16-bit and fp8 caches.
#include "attn_launch.hpp"

namespace hswd {

template <>
int32_t launch_attn_group<4, false>(const AttnParams& P, int mode, int D, int DT, int grid,
                                    hipStream_t st) {
    constexpr int G_ = 4;
    constexpr bool SH_ = false;
    HSWD_ATTN_CASE(256, kBF16) HSWD_ATTN_CASE(256, kF16) HSWD_ATTN_CASE(256, kFP8)
    HSWD_ATTN_CASE(128, kBF16) HSWD_ATTN_CASE(128, kF16) HSWD_ATTN_CASE(128, kFP8)
    return HSWD_ERR_UNSUPPORTED;
}

}  // namespace hswd
