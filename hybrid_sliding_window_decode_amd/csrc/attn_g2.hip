// Attention kernels with 2 query heads per kv head (grouped-query
// attention): head dims 256 and 128, 16-bit caches (a group of 2 over an
// fp8 cache runs the 4-head kernel).
#include "attn_launch.hpp"

namespace hswd {

template <>
int32_t launch_attn_group<2, false>(const AttnParams& P, int mode, int D, int DT, int grid,
                                    hipStream_t st) {
    constexpr int G_ = 2;
    constexpr bool SH_ = false;
    HSWD_ATTN_CASE(256, kBF16) HSWD_ATTN_CASE(256, kF16)
    HSWD_ATTN_CASE(128, kBF16) HSWD_ATTN_CASE(128, kF16)
    return HSWD_ERR_UNSUPPORTED;
}

}  // namespace hswd
