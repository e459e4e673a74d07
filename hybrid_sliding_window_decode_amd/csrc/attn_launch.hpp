// Launch of the attention kernel for one query-head group size G.  Each G
// has its own translation unit (attn_g1.hip, attn_g2.hip, attn_g4.hip,
// attn_g8.hip, and attn_g8s.hip for the pieces of larger groups), so the instantiations compile in parallel; hswd.hip picks one
// from H / Hkv.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/hswd.h"
#include "kernels/attn.hpp"

namespace hswd {

// Launches attn_kernel<D, T, ring, mode, G, SH> on `grid` workgroups.
// Returns HSWD_OK, HSWD_ERR_UNSUPPORTED when (D, T) has no instantiation for
// this (G, SH) (nothing is launched), or HSWD_ERR_HIP when the launch fails.
template <int G, bool SH>
int32_t launch_attn_group(const AttnParams& P, int mode, int D, int DT, int grid, hipStream_t st);
#define HSWD_DECLARE_GROUP(GV, SHV)                                                          \
    template <>                                                                             \
    int32_t launch_attn_group<GV, SHV>(const AttnParams& P, int mode, int D, int DT, int grid, \
                                       hipStream_t st);
HSWD_DECLARE_GROUP(1, false)
HSWD_DECLARE_GROUP(2, false)
HSWD_DECLARE_GROUP(4, false)
HSWD_DECLARE_GROUP(8, false)
HSWD_DECLARE_GROUP(8, true)
#undef HSWD_DECLARE_GROUP

template <int D, int DT, int G, bool SH>
int32_t launch_attn_dt(const AttnParams& P, int mode, int grid, hipStream_t st) {
    const dim3 g(grid), blk(kAttnThreads);
    if (P.ring) {
        if (mode == kModeStep) hipLaunchKernelGGL((attn_kernel<D, DT, true, kModeStep, G, SH>), g, blk, 0, st, P);
        else if (mode == kModeAttend) hipLaunchKernelGGL((attn_kernel<D, DT, true, kModeAttend, G, SH>), g, blk, 0, st, P);
        else hipLaunchKernelGGL((attn_kernel<D, DT, true, kModePartials, G, SH>), g, blk, 0, st, P);
    } else {
        if (mode == kModeStep) hipLaunchKernelGGL((attn_kernel<D, DT, false, kModeStep, G, SH>), g, blk, 0, st, P);
        else if (mode == kModeAttend) hipLaunchKernelGGL((attn_kernel<D, DT, false, kModeAttend, G, SH>), g, blk, 0, st, P);
        else hipLaunchKernelGGL((attn_kernel<D, DT, false, kModePartials, G, SH>), g, blk, 0, st, P);
    }
    return hipGetLastError() == hipSuccess ? HSWD_OK : HSWD_ERR_HIP;
}

}  // namespace hswd

// Body of launch_attn_group<G_, SH_> over a list of HSWD_ATTN_CASE(D, T) lines.
#define HSWD_ATTN_CASE(DV, TV) \
    if (D == DV && DT == TV) return launch_attn_dt<DV, TV, G_, SH_>(P, mode, grid, st);
