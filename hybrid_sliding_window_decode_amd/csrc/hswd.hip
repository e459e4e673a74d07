// libhswd: C ABI of hybrid sliding-window decode attention for gfx950.
// Host side: argument checks (before any launch), workspace layout, chunk
// count and work split, kernel dispatch.  Declarations and contracts: include/hswd.h.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/hswd.h"
#include "attn_launch.hpp"
#include "kernels/attn.hpp"
#include "kernels/small.hpp"

namespace {

using namespace hswd;

constexpr int kVersion = (0 << 16) | 7;
constexpr size_t kAlign = 256;
constexpr int kMaxChunkKeys = 2048;  // cap of the default keys per chunk
// Attention workgroups per CU the default split aims for: the residency of
// the largest kernels (up to 256 VGPRs per lane).  The smaller ones could
// hold more (the one-head bf16 kernel: 100 VGPRs, 34 KB of LDS), but more
// workgroups per (stream, kv head) measured slower (64 x 4096 bf16 full
// layer: 309 us at 512 workgroups, 334 us at 1024): each adds a partial to
// merge and splits a contiguous read.
constexpr int kWgsPerCu = 2;
// Longest position from which an append cache's launch takes the packed
// split (below it a launch is short, and the deal's extra round trip for the
// positions would show).
constexpr int kPackMinKeys = 32768;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int32_t launch_status() {
    return hipGetLastError() == hipSuccess ? HSWD_OK : HSWD_ERR_HIP;
}

// Workspace: [error word | counters (B*Hkv) | part_ml (B*H*n*2) | part_o (B*H*n*D)]
struct WsLayout {
    size_t counters, part_ml, part_o, total;
};

int32_t desc_check(const hswd_attn_desc* d) {
    if (!d) return HSWD_ERR_INVALID;
    if (d->batch < 0 || d->n_heads < 1 || d->n_kv_heads < 1 || d->n_slots < 1)
        return HSWD_ERR_INVALID;
    if (d->n_heads % d->n_kv_heads != 0) return HSWD_ERR_INVALID;
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
        return d->head_dim > 0 && d->head_dim % 8 == 0 ? HSWD_ERR_UNSUPPORTED : HSWD_ERR_INVALID;
    if (d->kv_dtype < HSWD_F32 || d->kv_dtype > HSWD_FP8_E4M3) return HSWD_ERR_INVALID;
    if (d->kv_dtype == HSWD_FP8_E4M3 && d->head_dim < 128) return HSWD_ERR_UNSUPPORTED;
    if (!(d->scale > 0.f) || !isfinite(d->scale)) return HSWD_ERR_INVALID;
    if (d->keys_per_split < 0 || d->chunks_per_workgroup < 0) return HSWD_ERR_INVALID;
    if (d->keys_per_split > 0 &&
        d->keys_per_split % chunk_quantum(d->head_dim, d->kv_dtype) != 0)
        return HSWD_ERR_INVALID;
    return HSWD_OK;
}

// An empty batch (B = 0, a valid descriptor otherwise) has nothing to
// compute: the entries return HSWD_OK without launching, whatever the
// pointers (an empty tensor may have none).
bool empty_batch(const hswd_attn_desc* d) {
    return d != nullptr && d->batch == 0 && desc_check(d) == HSWD_OK;
}

// Default keys per chunk of a ring (an append cache's streams take their
// own, auto_chunk_keys), from the cache geometry, element type and head
// grouping only (never the batch): 2^floor(log2(n_slots / 32)) clamped to
// [128, 512]; from 131072 rows on 2^floor(log2(n_slots / 128)), at most
// kMaxChunkKeys; and at least four quanta (a quantum, one tile per wave, is
// the keys of 32 KiB of K rows), so each wave scores four tiles per chunk
// end; grouped layers (H > Hkv) at least eight, since their stash holds a
// single chunk and every chunk end is a barrier.  Short caches get small
// chunks, so a small batch still spreads over many workgroups.  Long caches
// get longer chunks, so the last workgroup of a (stream, kv head) folds
// fewer partials, but not so long that a stream whose position is far below
// the capacity (the chunk follows the capacity, not the position) is left
// to a few workgroups: 8 x 131072 bf16 full layer 1280 us at 512-key chunks,
// 1249 at 1024, 1220 at 4096; one stream at position 5000 of that cache
// 19.0, 25.8 and 73.9 us.  The floor keeps the per-chunk reduction off the
// streaming rate (fp8 rows are half the bytes, so its chunks hold twice the
// keys).
int chunk_keys(const hswd_attn_desc* d) {
    if (d->keys_per_split > 0) return d->keys_per_split;
    int k = 128;
    while (k < 512 && (long)k * 2 * 32 <= d->n_slots) k *= 2;
    while (k < kMaxChunkKeys && (long)k * 2 * 128 <= d->n_slots) k *= 2;
    const int quanta = d->n_heads > d->n_kv_heads ? 8 : 4;
    const int floor_keys = quanta * chunk_quantum(d->head_dim, d->kv_dtype);
    if (k < floor_keys) k = floor_keys;
    // very long caches (past 2^23 rows at the cap): longer chunks still, so
    // the cache never needs more than kMaxChunks of them
    while ((d->n_slots + (long)k - 1) / k > kMaxChunks) k *= 2;
    return k;
}

// Append caches under the default chunking take each stream's chunk from
// its own valid keys (auto_chunk_keys: about 32 chunks of them), so a
// stream far below the capacity still spreads over many workgroups and a
// long one folds few partials; the chunk depends on the stream's position
// alone, never on the batch.  Rings and explicit chunk sizes keep one chunk
// for every stream.
bool auto_chunks(const hswd_attn_desc* d, int ring) { return !ring && d->keys_per_split == 0; }
int auto_floor(const hswd_attn_desc* d) {
    return (d->n_heads > d->n_kv_heads ? 8 : 4) * chunk_quantum(d->head_dim, d->kv_dtype);
}

// Chunks over the key range, the most any stream up to max_pos can have:
// a function of the cache geometry and max_pos only, never of the batch
// (the chunk size is part of the summation order).  auto_chunk_keys is
// nondecreasing, so ceil(n / chunk(n)) peaks where a range of constant chunk
// ends: at 32 * floor and below (32 chunks), at kAutoLongKeys - 1, at
// kAutoVeryLongKeys - 1, at the kMaxChunks threshold, or at max_pos itself.
int auto_chunks_of(int n, int fl, int hkv) {
    const int k = auto_chunk_keys(n, fl, hkv);
    return (int)((n + (long)k - 1) / k);
}
int num_chunks(const hswd_attn_desc* d, int ring, int max_pos) {
    const long keys = ring ? d->n_slots : (max_pos > 0 ? max_pos : 0);
    if (auto_chunks(d, ring)) {
        const int fl = auto_floor(d);
        const int hkv = d->n_kv_heads;
        const long ends[] = {keys, 32l * fl, kAutoLongKeys - 1l, kAutoVeryLongKeys - 1l,
                             (long)auto_very_long_cap(hkv) * kMaxChunks};
        int n = 1;
        for (long e : ends)
            if (e <= keys) n = max(n, auto_chunks_of((int)e, fl, hkv));
        return n;
    }
    const long K = chunk_keys(d);
    const long n = (keys + K - 1) / K;
    return n < 1 ? 1 : (int)n;
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
        v = 256;
    cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Chunks per workgroup: enough workgroups to fill the GPU once
// (kWgsPerCu per CU), each streaming as long a range as that allows.  Only
// the work split depends on this, never the arithmetic.
int chunks_per_workgroup(const hswd_attn_desc* d, int n_chunk) {
    if (d->chunks_per_workgroup > 0)
        return d->chunks_per_workgroup < n_chunk ? d->chunks_per_workgroup : n_chunk;
    const long pairs = (long)d->batch * d->n_kv_heads;
    const long target = (long)device_cus() * kWgsPerCu;
    long wpp = (target + pairs - 1) / pairs;
    if (wpp < 1) wpp = 1;
    if (wpp > n_chunk) wpp = n_chunk;
    return (int)((n_chunk + wpp - 1) / wpp);
}

// Query heads per kernel piece of a group (its kernel's G), and the pieces
// a group is split into.
int group_piece(int group, int DT) {
    (void)DT;
    if (group <= 2) return group;
    return group > 4 ? 8 : 4;
}
int group_pieces(const hswd_attn_desc* d) {
    const int group = d->n_heads / d->n_kv_heads;
    const int piece = group_piece(group, d->kv_dtype);
    return (group + piece - 1) / piece;
}

WsLayout ws_layout(const hswd_attn_desc* d, int n_chunk) {
    WsLayout L;
    const size_t pairs = (size_t)d->batch * d->n_kv_heads;
    const size_t bh = (size_t)d->batch * d->n_heads;
    const int np = group_pieces(d);
    // merge arrivals per (pair, piece), then entry arrivals per pair
    const size_t n_counters = pairs * np + (np > 1 ? pairs : 0);
    L.counters = kAlign;
    L.part_ml = L.counters + round_up(n_counters * sizeof(int32_t), kAlign);
    const size_t parts = n_chunk > 1 ? (size_t)n_chunk : 0;
    L.part_o = L.part_ml + round_up(bh * parts * 2 * sizeof(float), kAlign);
    L.total = L.part_o + round_up(bh * parts * d->head_dim * sizeof(float), kAlign);
    return L;
}

// Kernel launch for the descriptor's group size H / Hkv.  Groups of 1, 2,
// 4 and 8 query heads per kv head have their own kernels; a group of 3 runs
// the 4-head kernel with one head idle, 5 to 7 the 8-head kernel; a larger
// group is split into pieces of eight heads, one workgroup per piece in the
// same launch (each reads the cache; the last piece to finish writes the
// new entry).
template <int MODE>
int32_t dispatch_attn(AttnParams P, int D, int DT, int grid, hipStream_t st) {
    const int group = P.H / P.Hkv;
    P.Gq = group;
    if (group == 1) return launch_attn_group<1, false>(P, MODE, D, DT, grid, st);
    // A group of 2 over an fp8 cache runs the 4-head matrix-core kernel with
    // two heads idle: at 64 x 4096 its full layer takes 164.6 us against
    // 170.0 us for the 2-head kernel, its sliding layer ~27 us against 28.5.
    if (group == 2 && DT != kFP8)
        return launch_attn_group<2, false>(P, MODE, D, DT, grid, st);
    if (P.npiece > 1) return launch_attn_group<8, true>(P, MODE, D, DT, grid, st);
    return group_piece(group, DT) == 8 ? launch_attn_group<8, false>(P, MODE, D, DT, grid, st)
                                       : launch_attn_group<4, false>(P, MODE, D, DT, grid, st);
}

// Workspace of the entry point that allocates nothing: the library's own
// device array `scratch` (one per GPU, kept until the process ends).  Its
// layout is fixed, whatever the descriptor: error word, then a counter
// region of fixed size, then the chunk partials.  A call's partials never
// land on another call's counters, which every call leaves at zero.
constexpr size_t kScratchBytes = HSWD_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchCounterBytes = 64 * 1024;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

WsLayout noalloc_layout(const hswd_attn_desc* d, int n_chunk, bool partials) {
    WsLayout L;
    const size_t bh = (size_t)d->batch * d->n_heads;
    const size_t pairs = (size_t)d->batch * d->n_kv_heads;
    const int np = group_pieces(d);
    const size_t n_counters = pairs * np + (np > 1 ? pairs : 0);
    if (n_counters * sizeof(int32_t) > kScratchCounterBytes) {
        L.counters = L.part_ml = L.part_o = 0;
        L.total = SIZE_MAX;                       // more streams than the counters hold
        return L;
    }
    L.counters = kAlign;
    L.part_ml = L.counters + kScratchCounterBytes;
    const size_t parts = partials && n_chunk > 1 ? (size_t)n_chunk : 0;
    L.part_o = L.part_ml + round_up(bh * parts * 2 * sizeof(float), kAlign);
    L.total = L.part_o + round_up(bh * parts * d->head_dim * sizeof(float), kAlign);
    return L;
}

// Device address of `scratch` on the current device, looked up (and the
// array cleared by a fill kernel on `stream`) by the first call on that
// device.  In host code `scratch` names a host-side stand-in; only the
// address returned here may reach a kernel.
constexpr int kMaxDevices = 64;
struct ScratchDev {
    std::once_flag once;
    void* ptr = nullptr;
    int32_t status = HSWD_ERR_HIP;
};
ScratchDev g_scratch[kMaxDevices];

int32_t scratch_ptr(void** out, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HSWD_ERR_HIP;
    ScratchDev& sd = g_scratch[dev];
    std::call_once(sd.once, [&] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return;
        const size_t n = kScratchBytes / 4;
        hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0, stream,
                           static_cast<int32_t*>(p), n);
        if (hipGetLastError() != hipSuccess) return;
        sd.ptr = p;
        sd.status = HSWD_OK;
    });
    *out = sd.ptr;
    return sd.status;
}

// Shared argument checks and parameter set-up of the attention entries.
// scratch_ws: the workspace is the library's `scratch` array (ws is then
// its device address, and ws_bytes its size), in the fixed layout above.
int32_t attn_setup(AttnParams& P, int& grid, const hswd_attn_desc* d, int ring, int max_pos,
                   void* ws, size_t ws_bytes, bool need_ws, bool scratch_ws = false) {
    int32_t st = desc_check(d);
    if (st != HSWD_OK) return st;
    const int group = d->n_heads / d->n_kv_heads;       // query heads per kv head
    // grouped kernels: 16-bit and fp8 caches, head dim 128 or 256 (G query
    // vectors and accumulators per lane must fit beside the tiles in 256 VGPRs)
    if (group > 1 && (d->kv_dtype == HSWD_F32 || d->head_dim < 128)) return HSWD_ERR_UNSUPPORTED;
    // the kernels address a (stream, kv head) block with 32-bit offsets
    const size_t elt = d->kv_dtype == HSWD_F32 ? 4 : (d->kv_dtype == HSWD_FP8_E4M3 ? 1 : 2);
    if ((size_t)d->n_slots * d->head_dim * elt > 0xFFFFFFFFull) return HSWD_ERR_UNSUPPORTED;
    if (!ring) {
        if (max_pos < 0) return HSWD_ERR_INVALID;
        if ((long)max_pos + 1 > d->n_slots) return HSWD_ERR_CAPACITY;
    }
    const int n_chunk = num_chunks(d, ring, max_pos);
    if (n_chunk > kMaxChunks) return HSWD_ERR_INVALID;
    const bool autok = auto_chunks(d, ring);
    int cpw = chunks_per_workgroup(d, n_chunk);
    const int wpp = (n_chunk + cpw - 1) / cpw;
    // per-stream chunks: the launch's K and cpw are those of a stream at
    // max_pos (its chunks spread over the pair's wpp workgroups unless the
    // caller fixed the chunks per workgroup)
    const int K = autok ? auto_chunk_keys(max_pos, auto_floor(d), d->n_kv_heads) : chunk_keys(d);
    if (autok && d->chunks_per_workgroup == 0) {
        const int nb = max_pos > 0 ? (max_pos + K - 1) / K : 1;
        cpw = (nb + wpp - 1) / wpp;
    }
    if (need_ws) {
        if (!ws) return HSWD_ERR_WORKSPACE;
        if (!aligned16(ws)) return HSWD_ERR_ALIGN;
        // the scratch array holds chunk partials only when they cross
        // workgroups (the fused step folds them in place otherwise)
        const WsLayout L = scratch_ws ? noalloc_layout(d, n_chunk, wpp > 1) : ws_layout(d, n_chunk);
        if (ws_bytes < L.total) return HSWD_ERR_WORKSPACE;
        char* base = static_cast<char*>(ws);
        P.err = reinterpret_cast<int32_t*>(base);
        P.counters = reinterpret_cast<int32_t*>(base + L.counters);
        P.part_ml = reinterpret_cast<float*>(base + L.part_ml);
        P.part_o = reinterpret_cast<float*>(base + L.part_o);
    }
    P.B = d->batch;
    P.H = d->n_heads;
    P.Hkv = d->n_kv_heads;
    P.S = d->n_slots;
    P.K = K;
    P.auto_k = autok ? (d->chunks_per_workgroup == 0 ? 1 : 2) : 0;
    P.k_floor = auto_floor(d);
    P.n_chunk = n_chunk;
    P.cpw = cpw;
    P.wpp = wpp;
    P.ring = ring ? 1 : 0;
    P.max_pos = ring ? d->n_slots : max_pos;
    P.qscale = d->scale * 1.4426950408889634f;
    P.kv_scale = d->kv_scale;
    P.Gq = d->n_heads / d->n_kv_heads;
    P.npiece = group_pieces(d);
    // The packed split: long append caches under the default chunking (one
    // piece per group, at most one stream per thread of the deal) take their
    // workgroups from the positions on the device, from each stream's valid
    // keys (the fewest keys per workgroup whose workgroups fit in the pack),
    // instead of the same count for every stream: with ragged positions a
    // short stream's pair no longer holds workgroups idle while the long
    // ones stream.  Only the work split changes.
    P.pack = 0;
    if (autok && d->chunks_per_workgroup == 0 && wpp > 1 && P.npiece == 1 &&
        max_pos >= kPackMinKeys && d->batch <= kAttnThreads)
        P.pack = device_cus() * kWgsPerCu;
    grid = P.pack > 0 ? P.pack + d->batch * d->n_kv_heads
                      : d->batch * d->n_kv_heads * P.wpp * P.npiece;
    return HSWD_OK;
}

}  // namespace

extern "C" {

int32_t hswd_version(void) { return kVersion; }

const char* hswd_status_string(int32_t s) {
    switch (s) {
        case HSWD_OK: return "ok";
        case HSWD_ERR_INVALID: return "invalid argument";
        case HSWD_ERR_ALIGN: return "pointer not 16-byte aligned";
        case HSWD_ERR_WORKSPACE: return "workspace missing or too small";
        case HSWD_ERR_CAPACITY: return "position does not fit the cache";
        case HSWD_ERR_HIP: return "HIP runtime error";
        case HSWD_ERR_UNSUPPORTED: return "unsupported configuration";
        default: return "unknown status";
    }
}

size_t hswd_workspace_bytes(const hswd_attn_desc* d, int32_t ring, int32_t max_pos) {
    if (desc_check(d) != HSWD_OK) return 0;
    const int n = num_chunks(d, ring, max_pos);
    if (n > kMaxChunks) return 0;
    return ws_layout(d, n).total;
}

int32_t hswd_num_splits(const hswd_attn_desc* d, int32_t ring, int32_t max_pos) {
    int32_t st = desc_check(d);
    if (st != HSWD_OK) return st;
    const int n = num_chunks(d, ring, max_pos);
    return n > kMaxChunks ? HSWD_ERR_INVALID : n;
}

int32_t hswd_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws || ws_bytes < 4) return HSWD_ERR_WORKSPACE;
    if (!aligned16(ws)) return HSWD_ERR_ALIGN;
    const size_t n = ws_bytes / 4;
    const int grid = (int)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, as_stream(stream),
                       static_cast<int32_t*>(ws), n);
    return launch_status();
}

int32_t hswd_ring_mask(uint8_t* mask, int32_t* slot, const int32_t* pos, int32_t B,
                       int32_t n_slots, int32_t ring, void* stream) {
    if (B < 0 || n_slots < 1) return HSWD_ERR_INVALID;
    if (B == 0) return HSWD_OK;
    if (!pos || (!mask && !slot)) return HSWD_ERR_INVALID;
    hipLaunchKernelGGL(ring_mask_kernel, dim3(B), dim3(256), 0, as_stream(stream), mask, slot,
                       pos, n_slots, ring ? 1 : 0);
    return launch_status();
}

int32_t hswd_rope_apply(float* q, float* k, const int32_t* pos, int32_t B, int32_t H,
                        int32_t Hkv, int32_t D, int32_t rot_dim, double theta, void* stream) {
    if (B < 0 || H < 1 || D < 2 || (k && Hkv < 1)) return HSWD_ERR_INVALID;
    if (rot_dim <= 0 || rot_dim > D || (rot_dim & 1)) return HSWD_ERR_INVALID;
    if (!(theta > 0.0) || !isfinite(theta)) return HSWD_ERR_INVALID;
    const size_t lds = (size_t)D * sizeof(float);
    if (lds > 64 * 1024) return HSWD_ERR_UNSUPPORTED;
    const long vecs = (long)B * (H + (k ? Hkv : 0));
    if (vecs > 0x7fffffffL) return HSWD_ERR_UNSUPPORTED;
    if (B == 0) return HSWD_OK;
    if (!q || !pos) return HSWD_ERR_INVALID;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)vecs), dim3(256), lds, as_stream(stream), q, k,
                       pos, H, k ? Hkv : 0, D, rot_dim, log2(theta));
    return launch_status();
}

int32_t hswd_kv_slot_write(void* k_cache, void* v_cache, const float* k_rot, const float* v,
                           const int32_t* pos, const hswd_attn_desc* d, int32_t ring,
                           int32_t* slot_out, void* ws, void* stream) {
    int32_t st = desc_check(d);
    if (st != HSWD_OK) return st;
    if (d->batch == 0) return HSWD_OK;
    if (!k_cache || !v_cache || !k_rot || !v || !pos) return HSWD_ERR_INVALID;
    if (!ws) return HSWD_ERR_WORKSPACE;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_rot) || !aligned16(v) ||
        !aligned16(ws))
        return HSWD_ERR_ALIGN;
    const int grid = d->batch * d->n_kv_heads;
    hipStream_t s = as_stream(stream);
    int32_t* err = static_cast<int32_t*>(ws);
    const int ring01 = ring ? 1 : 0;
    switch (d->kv_dtype) {
        case HSWD_F32:
            hipLaunchKernelGGL(kv_write_kernel<kF32>, dim3(grid), dim3(256), 0, s, k_cache, v_cache,
                               k_rot, v, pos, d->n_kv_heads, d->n_slots, d->head_dim, ring01,
                               slot_out, err, d->kv_scale);
            break;
        case HSWD_F16:
            hipLaunchKernelGGL(kv_write_kernel<kF16>, dim3(grid), dim3(256), 0, s, k_cache, v_cache,
                               k_rot, v, pos, d->n_kv_heads, d->n_slots, d->head_dim, ring01,
                               slot_out, err, d->kv_scale);
            break;
        case HSWD_FP8_E4M3:
            hipLaunchKernelGGL(kv_write_kernel<kFP8>, dim3(grid), dim3(256), 0, s, k_cache, v_cache,
                               k_rot, v, pos, d->n_kv_heads, d->n_slots, d->head_dim, ring01,
                               slot_out, err, d->kv_scale);
            break;
        default:
            hipLaunchKernelGGL(kv_write_kernel<kBF16>, dim3(grid), dim3(256), 0, s, k_cache, v_cache,
                               k_rot, v, pos, d->n_kv_heads, d->n_slots, d->head_dim, ring01,
                               slot_out, err, d->kv_scale);
    }
    return launch_status();
}

static int32_t decode_attn(float* o, const float* q_rot, const float* k_rot, const float* v,
                           const void* kc, const void* vc, const int32_t* pos, int32_t ring,
                           int32_t max_pos, const hswd_attn_desc* d, void* ws, size_t ws_bytes,
                           void* stream) {
    if (empty_batch(d)) return HSWD_OK;
    if (!o || !q_rot || !k_rot || !v || !kc || !vc || !pos) return HSWD_ERR_INVALID;
    if (!aligned16(o) || !aligned16(q_rot) || !aligned16(k_rot) || !aligned16(v) ||
        !aligned16(kc) || !aligned16(vc))
        return HSWD_ERR_ALIGN;
    AttnParams P{};
    int grid = 0;
    int32_t st = attn_setup(P, grid, d, ring, max_pos, ws, ws_bytes, true);
    if (st != HSWD_OK) return st;
    P.out = o;
    P.q = q_rot;
    P.k = k_rot;
    P.v = v;
    P.kc = const_cast<void*>(kc);
    P.vc = const_cast<void*>(vc);
    P.pos = pos;
    return dispatch_attn<kModeAttend>(P, d->head_dim, d->kv_dtype, grid, as_stream(stream));
}

int32_t hswd_decode_attn_sliding(float* o, const float* q_rot, const float* k_rot,
                                 const float* v, const void* k_ring, const void* v_ring,
                                 const int32_t* pos, const hswd_attn_desc* d, void* ws,
                                 size_t ws_bytes, void* stream) {
    return decode_attn(o, q_rot, k_rot, v, k_ring, v_ring, pos, 1, 0, d, ws, ws_bytes, stream);
}

int32_t hswd_decode_attn_full(float* o, const float* q_rot, const float* k_rot,
                              const float* v, const void* k_cache, const void* v_cache,
                              const int32_t* pos, int32_t max_pos, const hswd_attn_desc* d,
                              void* ws, size_t ws_bytes, void* stream) {
    return decode_attn(o, q_rot, k_rot, v, k_cache, v_cache, pos, 0, max_pos, d, ws, ws_bytes,
                       stream);
}

int32_t hswd_decode_attn_partials(float* part_o, float* part_ml, const float* q_rot,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* pos, int32_t ring, int32_t max_pos,
                                  const hswd_attn_desc* d, void* stream) {
    if (empty_batch(d)) return HSWD_OK;
    if (!part_o || !part_ml || !q_rot || !k_cache || !v_cache || !pos) return HSWD_ERR_INVALID;
    if (!aligned16(part_o) || !aligned16(part_ml) || !aligned16(q_rot) || !aligned16(k_cache) ||
        !aligned16(v_cache))
        return HSWD_ERR_ALIGN;
    AttnParams P{};
    int grid = 0;
    int32_t st = attn_setup(P, grid, d, ring, max_pos, nullptr, 0, false);
    if (st != HSWD_OK) return st;
    // every chunk's partial is written, by the pairs' own workgroups
    P.pack = 0;
    grid = d->batch * d->n_kv_heads * P.wpp * P.npiece;
    P.q = q_rot;
    P.kc = const_cast<void*>(k_cache);
    P.vc = const_cast<void*>(v_cache);
    P.pos = pos;
    P.part_o = part_o;
    P.part_ml = part_ml;
    return dispatch_attn<kModePartials>(P, d->head_dim, d->kv_dtype, grid, as_stream(stream));
}

int32_t hswd_lse_merge(float* o, const float* part_o, const float* part_ml, int32_t B,
                       int32_t H, int32_t D, int32_t n, void* stream) {
    if (B < 0 || H < 1 || D < 1 || n < 1) return HSWD_ERR_INVALID;
    if (n > 1024) return HSWD_ERR_UNSUPPORTED;
    if (B == 0) return HSWD_OK;
    if (!o || !part_o || !part_ml) return HSWD_ERR_INVALID;
    hipLaunchKernelGGL(lse_merge_kernel, dim3(B * H), dim3(256), 0, as_stream(stream), o, part_o,
                       part_ml, D, n);
    return launch_status();
}

int32_t hswd_head_gate(float* out, const float* o, const float* gate, int32_t B, int32_t H,
                       int32_t D, void* stream) {
    if (B < 0 || H < 1 || D < 1) return HSWD_ERR_INVALID;
    if (B == 0) return HSWD_OK;
    if (!out || !o || !gate) return HSWD_ERR_INVALID;
    hipLaunchKernelGGL(head_gate_kernel, dim3(B * H), dim3(256), 0, as_stream(stream), out, o,
                       gate, D);
    return launch_status();
}

static int32_t layer_step(float* out, const float* q, const float* k, const float* v,
                          const float* gate, const float* gx, const float* gw, int32_t hidden,
                          void* k_cache, void* v_cache, const int32_t* pos, int32_t ring,
                          int32_t rot_dim, double theta, int32_t max_pos,
                          const hswd_attn_desc* d, void* ws, size_t ws_bytes, void* stream,
                          bool noalloc = false, int32_t* err = nullptr) {
    if (!d || rot_dim <= 0 || rot_dim > d->head_dim || (rot_dim & 1)) return HSWD_ERR_INVALID;
    if (!(theta > 0.0) || !isfinite(theta)) return HSWD_ERR_INVALID;
    if (empty_batch(d)) return HSWD_OK;
    if (!out || !q || !k || !v || !k_cache || !v_cache || !pos) return HSWD_ERR_INVALID;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v) ||
        !aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)err & 3u) != 0)
        return HSWD_ERR_ALIGN;
    AttnParams P{};
    int grid = 0;
    int32_t st;
    if (noalloc) {
        // the size check first, on a stand-in base: a refused call touches
        // no device state
        st = attn_setup(P, grid, d, ring, max_pos, reinterpret_cast<void*>(kAlign), kScratchBytes,
                        true, true);
        if (st != HSWD_OK) return st;
        st = scratch_ptr(&ws, as_stream(stream));
        if (st != HSWD_OK) return st;
        ws_bytes = kScratchBytes;
    }
    st = attn_setup(P, grid, d, ring, max_pos, ws, ws_bytes, true, noalloc);
    if (st != HSWD_OK) return st;
    if (err) P.err = err;
    P.out = out;
    P.q = q;
    P.k = k;
    P.v = v;
    P.gate = gate;
    P.gx = gx;
    P.gw = gw;
    P.hidden = hidden;
    P.kc = k_cache;
    P.vc = v_cache;
    P.pos = pos;
    P.rot = rot_dim;
    P.log2_theta = log2(theta);
    return dispatch_attn<kModeStep>(P, d->head_dim, d->kv_dtype, grid, as_stream(stream));
}

int32_t hswd_layer_step(float* out, const float* q, const float* k, const float* v,
                        const float* gate, void* k_cache, void* v_cache, const int32_t* pos,
                        int32_t ring, int32_t rot_dim, double theta, int32_t max_pos,
                        const hswd_attn_desc* d, void* ws, size_t ws_bytes, void* stream) {
    return layer_step(out, q, k, v, gate, nullptr, nullptr, 0, k_cache, v_cache, pos, ring,
                      rot_dim, theta, max_pos, d, ws, ws_bytes, stream);
}

int32_t hswd_layer_step_noalloc(float* out, const float* q, const float* k, const float* v,
                                const float* gate, void* k_cache, void* v_cache,
                                const int32_t* pos, int32_t ring, int32_t rot_dim, double theta,
                                int32_t max_pos, const hswd_attn_desc* d, int32_t* err,
                                void* stream) {
    return layer_step(out, q, k, v, gate, nullptr, nullptr, 0, k_cache, v_cache, pos, ring,
                      rot_dim, theta, max_pos, d, nullptr, 0, stream, true, err);
}

int32_t hswd_layer_step_gproj(float* out, const float* q, const float* k, const float* v,
                              const float* x, const float* w_g, int32_t hidden, void* k_cache,
                              void* v_cache, const int32_t* pos, int32_t ring, int32_t rot_dim,
                              double theta, int32_t max_pos, const hswd_attn_desc* d, void* ws,
                              size_t ws_bytes, void* stream) {
    if (hidden < 1) return HSWD_ERR_INVALID;
    if (!(d && d->batch == 0) && (!x || !w_g)) return HSWD_ERR_INVALID;
    return layer_step(out, q, k, v, nullptr, x, w_g, hidden, k_cache, v_cache, pos, ring,
                      rot_dim, theta, max_pos, d, ws, ws_bytes, stream);
}

int32_t hswd_gate_proj(float* logits, const float* x, const float* w_g, int32_t B,
                       int32_t hidden, int32_t H, void* stream) {
    if (B < 0 || hidden < 1 || H < 1) return HSWD_ERR_INVALID;
    if (B == 0) return HSWD_OK;
    if (!logits || !x || !w_g) return HSWD_ERR_INVALID;
    hipLaunchKernelGGL(gate_proj_kernel, dim3(B * H), dim3(256), 0, as_stream(stream), logits, x,
                       w_g, hidden, H);
    return launch_status();
}

int32_t hswd_check_errors(const void* ws, int32_t* flags_out, void* stream) {
    if (!ws) return HSWD_ERR_WORKSPACE;
    int32_t flags = 0;
    if (hipMemcpyAsync(&flags, ws, sizeof(int32_t), hipMemcpyDeviceToHost, as_stream(stream)) !=
        hipSuccess)
        return HSWD_ERR_HIP;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return HSWD_ERR_HIP;
    if (flags_out) *flags_out = flags;
    return flags ? HSWD_ERR_CAPACITY : HSWD_OK;
}

}  // extern "C"
