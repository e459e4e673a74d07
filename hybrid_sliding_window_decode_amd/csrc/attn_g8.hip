// Attention kernels with 8 query heads per kv head (grouped-query attention,
// 5 to 8 heads) over fp8, bf16 and f16 caches: head dims 256 and 128, scores
// and the value product on the matrix cores.
#include "attn_launch.hpp"

namespace hswd {

template <>
int32_t launch_attn_group<8, false>(const AttnParams& P, int mode, int D, int DT, int grid,
                                    hipStream_t st) {
    constexpr int G_ = 8;
    constexpr bool SH_ = false;
    HSWD_ATTN_CASE(256, kFP8) HSWD_ATTN_CASE(128, kFP8)
    HSWD_ATTN_CASE(256, kBF16) HSWD_ATTN_CASE(256, kF16)
    HSWD_ATTN_CASE(128, kBF16) HSWD_ATTN_CASE(128, kF16)
    return HSWD_ERR_UNSUPPORTED;
}

}  // namespace hswd
