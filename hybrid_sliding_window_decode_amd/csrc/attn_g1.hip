// Attention kernels with one query head per kv head (H = Hkv): every head
// dim and cache type the library supports.
#include "attn_launch.hpp"

namespace hswd {

template <>
int32_t launch_attn_group<1, false>(const AttnParams& P, int mode, int D, int DT, int grid,
                                    hipStream_t st) {
    constexpr int G_ = 1;
    constexpr bool SH_ = false;
    HSWD_ATTN_CASE(256, kBF16) HSWD_ATTN_CASE(256, kF16) HSWD_ATTN_CASE(256, kF32)
    HSWD_ATTN_CASE(128, kBF16) HSWD_ATTN_CASE(128, kF16) HSWD_ATTN_CASE(128, kF32)
    HSWD_ATTN_CASE(64, kBF16) HSWD_ATTN_CASE(64, kF16) HSWD_ATTN_CASE(64, kF32)
    HSWD_ATTN_CASE(256, kFP8) HSWD_ATTN_CASE(128, kFP8)
    return HSWD_ERR_UNSUPPORTED;
}

}  // namespace hswd
