// The per-token kernels around the attention: RoPE, slot/mask, entry write,
// head gate, split merge, workspace fill.  Each moves a few KiB per stream.
#pragma once

#include "common.hpp"

namespace hswd {

// RoPE in place, one workgroup per (stream, head vector): q [B,H,D] heads
// first, then k [B,Hkv,D].  Each thread rotates whole elements; both
// members of a pair are computed from the unrotated vector before any store
// (the block barrier), through D floats of LDS.
__global__ __launch_bounds__(256) void rope_kernel(float* q, float* k, const int32_t* pos, int H,
                                                   int Hkv, int D, int rot, double log2_theta) {
    extern __shared__ float sm[];                // D rotated values
    const int nvec = H + Hkv;
    const int b = blockIdx.x / nvec;
    const int v = blockIdx.x % nvec;
    const int p = pos[b];
    float* x = v < H ? q + ((size_t)b * H + v) * D : k + ((size_t)b * Hkv + (v - H)) * D;
    for (int i = threadIdx.x; i < D; i += blockDim.x) sm[i] = rope_elem(x, i, rot, log2_theta, p);
    __syncthreads();
    for (int i = threadIdx.x; i < D; i += blockDim.x) x[i] = sm[i];
}

// Slot and mask of each stream.
__global__ __launch_bounds__(256) void ring_mask_kernel(uint8_t* mask, int32_t* slot,
                                                        const int32_t* pos, int S, int ring) {
    const int b = blockIdx.x;
    const int p = pos[b];
    const int nv = p < 0 ? 0 : (p < S ? p : S);
    if (mask)
        for (int s = threadIdx.x; s < S; s += blockDim.x) mask[(size_t)b * S + s] = s < nv;
    if (slot && threadIdx.x == 0) slot[b] = p < 0 ? -1 : (ring ? p % S : p);
}

// Round the new entry to the cache element type and store it, one workgroup
// per (stream, kv head).
template <int DT>
__global__ __launch_bounds__(256) void kv_write_kernel(void* kc, void* vc, const float* k,
                                                       const float* v, const int32_t* pos,
                                                       int Hkv, int S, int D, int ring,
                                                       int32_t* slot_out, int32_t* err,
                                                       const float* kv_scale) {
    using St = typename Storage<DT>::type;
    const int pair = blockIdx.x;
    const int b = pair / Hkv;
    const int p = pos[b];
    int row = -1;
    if (p >= 0) {
        if (ring) row = p % S;
        else if (p < S) row = p;
    }
    if (threadIdx.x == 0 && pair % Hkv == 0) {
        if (slot_out) slot_out[b] = row;
        if (p < 0) atomicOr(err, 4);
        else if (row < 0) atomicOr(err, 1);
    }
    if (row < 0) return;
    St* kd = reinterpret_cast<St*>(kc) + ((size_t)pair * S + row) * D;
    St* vd = reinterpret_cast<St*>(vc) + ((size_t)pair * S + row) * D;
    if constexpr (DT == kFP8) {     // the code of x / scale (quotient rounded to float32)
        const int g = pair % Hkv;
        const float ks = kv_scale ? kv_scale[g] : 1.f, vs = kv_scale ? kv_scale[Hkv + g] : 1.f;
        for (int t = threadIdx.x; t < D; t += blockDim.x) {
            kd[t] = round_to_elt<DT>(__fdiv_rn(k[(size_t)pair * D + t], ks));
            vd[t] = round_to_elt<DT>(__fdiv_rn(v[(size_t)pair * D + t], vs));
        }
    } else {
        for (int t = threadIdx.x; t < D; t += blockDim.x) {
            kd[t] = round_to_elt<DT>(k[(size_t)pair * D + t]);
            vd[t] = round_to_elt<DT>(v[(size_t)pair * D + t]);
        }
    }
}

// out = o * sigmoid(gate), one workgroup per (stream, head).
__global__ __launch_bounds__(256) void head_gate_kernel(float* out, const float* o,
                                                        const float* gate, int D) {
    const int bh = blockIdx.x;
    const float s = 1.f / (1.f + expf(-gate[bh]));
    for (int t = threadIdx.x; t < D; t += blockDim.x) out[(size_t)bh * D + t] = o[(size_t)bh * D + t] * s;
}

// Gate logits: logits[b][h] = x[b] . w_g[h], one workgroup of 256
// threads per (stream, head) (the same sum as the fused layer step).
__global__ __launch_bounds__(256) void gate_proj_kernel(float* logits, const float* x,
                                                        const float* w, int hidden, int H) {
    __shared__ float sm[4];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    float gs = gate_share(x + (size_t)b * hidden, w + (size_t)h * hidden, hidden, tid, 256);
    gs = wave_sum(gs);
    if ((tid & 63) == 0) sm[tid >> 6] = gs;
    __syncthreads();
    if (tid == 0) logits[bh] = lds_tree_sum<4>(sm);
}

// Merge n partials (natural-log m, l, unnormalised o) of each (stream, head).
__global__ __launch_bounds__(256) void lse_merge_kernel(float* out, const float* part_o,
                                                        const float* part_ml, int D, int n) {
    __shared__ float sm_w[1024];
    __shared__ float sm_red[4];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const float* ml = part_ml + (size_t)bh * n * 2;
    const float kLog2e = 1.4426950408889634f;
    float mloc = -INFINITY;
    for (int i = tid; i < n; i += 256) {
        const float mi = ml[2 * i] * kLog2e, li = ml[2 * i + 1];
        sm_w[i] = li > 0.f ? mi : -INFINITY;
        mloc = fmaxf(mloc, sm_w[i]);
    }
    mloc = wave_max(mloc);
    if (lane == 0) sm_red[wid] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(sm_red[0], sm_red[1]), fmaxf(sm_red[2], sm_red[3]));
    __syncthreads();
    float lloc = 0.f;
    for (int i = tid; i < n; i += 256) {
        const float wi = M == -INFINITY ? 0.f : fast_exp2(sm_w[i] - M);
        sm_w[i] = wi;
        lloc = fmaf(ml[2 * i + 1], wi, lloc);
    }
    lloc = wave_sum(lloc);
    if (lane == 0) sm_red[wid] = lloc;
    __syncthreads();
    const float L = (sm_red[0] + sm_red[1]) + (sm_red[2] + sm_red[3]);
    for (int t = tid; t < D; t += 256) {
        const float* po = part_o + (size_t)bh * n * D + t;
        float acc = 0.f;
        int i = 0;
        for (; i + 16 <= n; i += 16) {              // 16 loads in flight, then fold
            float x[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) x[u] = po[(size_t)(i + u) * D];
#pragma unroll
            for (int u = 0; u < 16; ++u) acc = fmaf(x[u], sm_w[i + u], acc);
        }
        for (; i < n; ++i) acc = fmaf(po[(size_t)i * D], sm_w[i], acc);
        out[(size_t)bh * D + t] = acc / L;
    }
}

// Zero n 32-bit words.
__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

}  // namespace hswd
