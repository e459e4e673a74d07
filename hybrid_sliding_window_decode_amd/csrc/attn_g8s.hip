// Attention kernels with 8 query heads per kv head for the pieces of a
// larger group (several workgroups read each row, so the rows are loaded
// without the streaming hint): fp8, bf16 and f16 caches, head dims 256 and
// 128.
#include "attn_launch.hpp"

namespace hswd {

template <>
int32_t launch_attn_group<8, true>(const AttnParams& P, int mode, int D, int DT, int grid,
                                   hipStream_t st) {
    constexpr int G_ = 8;
    constexpr bool SH_ = true;
    HSWD_ATTN_CASE(256, kFP8) HSWD_ATTN_CASE(128, kFP8)
    HSWD_ATTN_CASE(256, kBF16) HSWD_ATTN_CASE(256, kF16)
    HSWD_ATTN_CASE(128, kBF16) HSWD_ATTN_CASE(128, kF16)
    return HSWD_ERR_UNSUPPORTED;
}

}  // namespace hswd
