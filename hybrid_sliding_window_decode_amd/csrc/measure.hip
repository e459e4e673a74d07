// libhswd_measure.so: the streaming-read probe the benchmark compares the
// attention kernels with (include/hswd_measure.h).  Not part of the decode
// path, so it lives outside libhswd.so.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/hswd.h"
#include "../../include/hswd_measure.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Read n16 16-byte words once, each workgroup a contiguous range, eight
// non-temporal 128-bit loads in flight per thread.  The loaded words are
// folded into a value that is stored only in the (practically impossible)
// case that it equals a fixed pattern, so the loads cannot be dropped and
// nothing else reaches memory.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* p, size_t n16,
                                                          uint32_t* sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t beg = per * blockIdx.x;
    const size_t end = beg + per < n16 ? beg + per : n16;
    uint32_t acc = 0;
    size_t i = beg + threadIdx.x;
    for (; i + 7 * 256 < end; i += 8 * 256) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += 256) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

bool aligned16(const void* q) { return ((uintptr_t)q & 15u) == 0; }

}  // namespace

extern "C" int32_t hswd_measure_stream_read(const void* buf, size_t bytes, void* sink,
                                            int32_t workgroups, void* stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536)
        return HSWD_ERR_INVALID;
    if (!aligned16(buf) || !aligned16(sink)) return HSWD_ERR_ALIGN;
    hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                       bytes / 16, static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? HSWD_OK : HSWD_ERR_HIP;
}
