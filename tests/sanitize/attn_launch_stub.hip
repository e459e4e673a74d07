// Test infrastructure: the attention launchers of libhswd replaced by stubs
// that launch nothing and report HSWD_ERR_HIP (what a host without a GPU
// returns), so the host side of the library (hswd.hip: argument checks,
// chunking, workspace layout, dispatch) can be built with sanitizers without
// compiling the attention kernels.
#include "../../hybrid_sliding_window_decode_amd/csrc/attn_launch.hpp"

namespace hswd {
#define HSWD_STUB_GROUP(GV, SHV)                                                              \
    template <>                                                                              \
    int32_t launch_attn_group<GV, SHV>(const AttnParams&, int, int, int, int, hipStream_t) { \
        return HSWD_ERR_HIP;                                                                 \
    }
HSWD_STUB_GROUP(1, false)
HSWD_STUB_GROUP(2, false)
HSWD_STUB_GROUP(4, false)
HSWD_STUB_GROUP(8, false)
HSWD_STUB_GROUP(8, true)
#undef HSWD_STUB_GROUP
}  // namespace hswd
