// Decode attention over a ring or an append KV cache, split over the key
// range, with the new entry joined in score space.
//
// One workgroup (4 waves) per (stream, kv head, key split).  The cache is
// streamed once from HBM: each wave reads whole 16-key (bf16/f16) or 8-key
// (f32) tiles with 128-bit loads, one cache row per 32 (or 64) lanes, lanes
// over head dims, and keeps the next tile's loads in flight while it scores
// the current one (register double buffering).  Dot products are reduced
// across lanes with a transposed butterfly (each exchange halves the keys a
// lane carries), so the cross-lane cost is about one exchange per key.  The
// softmax is online (running max and sum per wave), in base 2 with the
// log2(e) folded into the query scale.  The four waves' partials are merged
// through LDS into one partial per workgroup; with several splits the last
// workgroup of a (stream, kv head) to arrive -- counted with an atomic --
// merges all of them, joins the new entry as a one-key partial, applies the
// gate and, in the fused layer step, writes the entry into the cache after
// every read of that cache block has finished.
//
// Sources: vLLM-Omni fork commit log, score-space join commit (join scores,
// not keys; ring without reordering, only a mask; 511 slots) and Spark-X2.5
// model commit (per-type RoPE, sigmoid head gate); TensorFold pull request
// 608 review thread (split the key range to fill the GPU, merge partials,
// keep tiles in flight, issue the merge's loads before folding); pega-omni
// pull request 4 (RoPE, ring write and attention in one launch).
#pragma once

#include "common.hpp"

namespace hswd {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int kMaxSplits = 1024;

// What a launch of the attention kernel produces.
enum AttnMode : int {
    kModeAttend = 0,    // o = attention output before the gate (q, k already rotated)
    kModeStep = 1,      // whole layer step: rope, attend, gate, write the entry
    kModePartials = 2,  // split partials of the cached keys only (natural-log m)
};

struct AttnParams {
    float* out;              // [B,H,D]
    const float* q;          // [B,H,D]: rotated (attend) or raw (step)
    const float* k;          // [B,Hkv,D]: rotated (attend) or raw (step); unused for partials
    const float* v;          // [B,Hkv,D]
    const float* gate;       // [B,H] or null
    void* kc;                // cache [B,Hkv,S,D]
    void* vc;
    const int32_t* pos;      // [B]
    float* part_o;           // partials [B*H][n_split][D]
    float* part_ml;          // [B*H][n_split][2]
    int32_t* counters;       // [B*Hkv]
    int32_t* err;            // error word
    int B, H, Hkv, S;        // S: ring slots or append capacity
    int kps;                 // keys per split
    int n_split;
    int ring;
    int max_pos;             // append: host bound of pos (grid size)
    int rot;
    double log2_theta;
    float qscale;            // softmax scale * log2(e)
};

template <int D, int DT>
struct AttnGeo {
    static constexpr int EB = DT == kF32 ? 4 : 2;     // element bytes
    static constexpr int EPC = 16 / EB;               // elements per 16-byte chunk
    static constexpr int LPR = D / EPC;               // lanes per cache row
    static constexpr int RPI = kWave / LPR;           // rows per wave-wide load
    static constexpr int NL = 8;                      // loads per tile (K and V each)
    static constexpr int KT = NL * RPI;               // keys per wave tile
    static constexpr int STEP = LPR / NL;             // lane stride between reduced keys
    static_assert(LPR >= NL && LPR <= kWave && kWave % LPR == 0, "geometry");
};

// One exchange of the transposed butterfly: a lane whose `M` bit is set
// keeps its upper value and sends its lower one; its partner does the
// opposite, so each keeps the sum over both lanes of one of the two keys.
template <int M>
__device__ __forceinline__ float tstage(float lo, float hi, bool up) {
    const float send = up ? lo : hi;
    const float keep = up ? hi : lo;
    return keep + xor_lane<M>(send);
}

// Sum over the LPR lanes that share a cache row of eight per-load partials
// (v[i] = this lane's partial dot product for load i), spreading the eight
// sums over the lanes: on exit this lane holds the full sum for load
// ((lane % LPR) / (LPR / 8)).  Seven exchanges for eight keys instead of
// log2(LPR) per key.  Written on scalars so every select stays in registers.
template <int LPR>
__device__ __forceinline__ float transposed_reduce8(const float (&v)[8], int lane) {
    constexpr int M1 = LPR / 2, M2 = LPR / 4, M3 = LPR / 8;
    bool u = (lane & M1) != 0;
    const float a0 = tstage<M1>(v[0], v[4], u), a1 = tstage<M1>(v[1], v[5], u);
    const float a2 = tstage<M1>(v[2], v[6], u), a3 = tstage<M1>(v[3], v[7], u);
    u = (lane & M2) != 0;
    const float b0 = tstage<M2>(a0, a2, u), b1 = tstage<M2>(a1, a3, u);
    u = (lane & M3) != 0;
    float c = tstage<M3>(b0, b1, u);
    // the remaining lane bits below M3 hold copies of the same key: plain sum
#pragma unroll
    for (int m = M3 / 2; m >= 1; m >>= 1) c += xor_lane_rt(c, m);
    return c;
}

template <int D, int DT, bool RING, int MODE>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnParams P) {
    using G = AttnGeo<D, DT>;
    using S = typename Storage<DT>::type;
    constexpr int EPC = G::EPC, LPR = G::LPR, RPI = G::RPI, NL = G::NL, KT = G::KT;

    __shared__ float sm_q[D];
    __shared__ float sm_o[kAttnWaves][D];
    __shared__ float sm_m[kAttnWaves], sm_l[kAttnWaves];
    __shared__ float sm_red[kAttnWaves];
    __shared__ float sm_dot[kAttnWaves];
    __shared__ float sm_w[kMaxSplits];
    __shared__ int sm_last;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;

    // Workgroup -> (stream, kv head, split).  When the pair count allows, the
    // splits of one pair go to the same XCD (workgroups are dealt to the 8
    // XCDs round robin), so the merging workgroup finds them in its L2.
    const int n_pairs = P.B * P.Hkv;
    int pair, split;
    {
        const int w = blockIdx.x;
        if ((n_pairs & 7) == 0 && P.n_split > 1) {
            const int k = w >> 3;
            pair = (k / P.n_split) * 8 + (w & 7);
            split = k % P.n_split;
        } else {
            pair = w / P.n_split;
            split = w % P.n_split;
        }
    }
    const int b = pair / P.Hkv;
    const int g = pair % P.Hkv;
    const int h = g;                       // one query head per kv head
    const int bh = b * P.H + h;
    const int p = P.pos[b];

    // Valid cache rows: ring slots s < min(p, S); append rows < p.
    int nv = p < 0 ? 0 : (p < P.S ? p : P.S);
    if (!RING) {
        const int grid_keys = P.n_split * P.kps;
        if (nv > grid_keys) nv = grid_keys;
        if (MODE != kModePartials && split == 0 && g == 0 && tid == 0 && p > P.max_pos)
            atomicOr(P.err, 2);
    }
    if (MODE != kModePartials && split == 0 && g == 0 && tid == 0 && p < 0) atomicOr(P.err, 4);

    // Query (rotated in-kernel for the fused step), scaled by scale*log2(e).
    {
        const float* qv = P.q + (size_t)bh * D;
        for (int t = tid; t < D; t += kAttnThreads) {
            float x = MODE == kModeStep ? rope_elem(qv, t, P.rot, P.log2_theta, p) : qv[t];
            sm_q[t] = x * P.qscale;
        }
    }
    __syncthreads();

    const int c = lane % LPR;       // 16-byte chunk of the row this lane reads
    const int r = lane / LPR;       // row within a wave-wide load
    float qs[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) qs[e] = sm_q[c * EPC + e];

    const int j0 = split * P.kps;
    int j1 = j0 + P.kps;
    if (j1 > nv) j1 = nv;
    const int n_keys = j1 > j0 ? j1 - j0 : 0;
    const int n_tiles = (n_keys + KT - 1) / KT;
    const int my_n = n_tiles > wid ? (n_tiles - wid + kAttnWaves - 1) / kAttnWaves : 0;

    const S* kbase = reinterpret_cast<const S*>(P.kc) + (size_t)pair * P.S * D + c * EPC;
    const S* vbase = reinterpret_cast<const S*>(P.vc) + (size_t)pair * P.S * D + c * EPC;

    float m_run = -INFINITY;
    float l_lane = 0.f;
    float o_acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) o_acc[e] = 0.f;

    uint4 kA[NL], vA[NL], kB[NL], vB[NL];

    // Tile j of this wave covers keys j0 + (wid + 4j) * KT ...; rows past the
    // valid range are clamped onto the last valid row (never reading an
    // unwritten slot) and masked out of the softmax.
    auto load_tile = [&](uint4 (&kt)[NL], uint4 (&vt)[NL], int j) {
        const int base = j0 + (wid + kAttnWaves * j) * KT + r;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            int row = base + i * RPI;
            row = row < j1 ? row : j1 - 1;
            kt[i] = *reinterpret_cast<const uint4*>(kbase + (size_t)row * D);
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            int row = base + i * RPI;
            row = row < j1 ? row : j1 - 1;
            vt[i] = *reinterpret_cast<const uint4*>(vbase + (size_t)row * D);
        }
    };

    auto compute_tile = [&](const uint4 (&kt)[NL], const uint4 (&vt)[NL], int j) {
        const int tile0 = j0 + (wid + kAttnWaves * j) * KT;
        float part[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            float kf[EPC];
            unpack16<DT>(kt[i], kf);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) acc = fmaf(qs[e], kf[e], acc);
            part[i] = acc;
        }
        static_assert(NL == 8, "tile of eight loads");
        float s = transposed_reduce8<LPR>(part, lane);
        const int ki = (lane % LPR) / G::STEP;          // load index of this lane's key
        const int key = tile0 + ki * RPI + r;
        s = key < j1 ? s : -INFINITY;
        // tile max over the distinct keys (lane bits >= STEP)
        float mx = s;
#pragma unroll
        for (int m = G::STEP; m < kWave; m <<= 1) mx = fmaxf(mx, xor_lane_rt(mx, m));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        const float pr = fast_exp2(s - m_new);
        m_run = m_new;
        l_lane = l_lane * alpha + ((lane & (G::STEP - 1)) == 0 ? pr : 0.f);
#pragma unroll
        for (int e = 0; e < EPC; ++e) o_acc[e] *= alpha;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const float pi = lane_value(pr, r * LPR + i * G::STEP);
            float vf[EPC];
            unpack16<DT>(vt[i], vf);
#pragma unroll
            for (int e = 0; e < EPC; ++e) o_acc[e] = fmaf(pi, vf[e], o_acc[e]);
        }
    };

    if (my_n > 0) load_tile(kA, vA, 0);
    int j = 0;
    for (; j + 2 < my_n; j += 2) {
        load_tile(kB, vB, j + 1);
        compute_tile(kA, vA, j);
        load_tile(kA, vA, j + 2);
        compute_tile(kB, vB, j + 1);
    }
    if (j + 1 < my_n) {
        load_tile(kB, vB, j + 1);
        compute_tile(kA, vA, j);
        compute_tile(kB, vB, j + 1);
    } else if (j < my_n) {
        compute_tile(kA, vA, j);
    }

    // Wave partial: l over all lanes (one copy per key counted), o summed over
    // the rows a wave-wide load spans.
    const float l_w = wave_sum(l_lane);
#pragma unroll
    for (int m = LPR; m < kWave; m <<= 1) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) o_acc[e] += xor_lane_rt(o_acc[e], m);
    }
    if (r == 0) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) sm_o[wid][c * EPC + e] = o_acc[e];
    }
    if (lane == 0) {
        sm_m[wid] = m_run;
        sm_l[wid] = l_w;
    }
    __syncthreads();

    // Workgroup partial (base-2 max M, sum L, unnormalised o) for dim t.
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm_m[w]);
    float L = 0.f;
    float o_t = 0.f;
    const int t = tid;                       // this thread's head dim (t < D)
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float a = fast_exp2(sm_m[w] - M);
            L = fmaf(sm_l[w], a, L);
            if (t < D) o_t = fmaf(sm_o[w][t], a, o_t);
        }
    }

    if (MODE == kModePartials) {
        const size_t idx = (size_t)bh * P.n_split + split;
        if (t < D) P.part_o[idx * D + t] = o_t;
        if (tid == 0) {
            P.part_ml[idx * 2 + 0] = M == -INFINITY ? -INFINITY : M * 0.69314718055994531f;
            P.part_ml[idx * 2 + 1] = L;
        }
        return;
    }

    if (P.n_split > 1) {
        // Partials cross workgroups (and possibly XCDs).  They are written and
        // read only with agent-scope atomic stores and loads, which go to the
        // device-coherent level themselves, so no L2 write-back or invalidate
        // is needed: each thread waits for its own stores to complete, the
        // barrier makes that true for the whole workgroup, and only then is
        // the arrival counted.  The merging workgroup reads the partials after
        // it has seen the final count.
        const size_t idx = (size_t)bh * P.n_split + split;
        if (t < D) st_agent(P.part_o + idx * D + t, o_t);
        if (tid == 0) {
            st_agent(P.part_ml + idx * 2 + 0, M);
            st_agent(P.part_ml + idx * 2 + 1, L);
        }
        wait_stores_complete();
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(&P.counters[pair], 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            sm_last = prev == P.n_split - 1;
        }
        __syncthreads();
        if (!sm_last) return;

        // Last arrival merges every split of this (stream, head).
        const float* pml = P.part_ml + (size_t)bh * P.n_split * 2;
        float mloc = -INFINITY;
        for (int i = tid; i < P.n_split; i += kAttnThreads) {
            const float mi = ld_agent(pml + 2 * i);
            const float li = ld_agent(pml + 2 * i + 1);
            sm_w[i] = li > 0.f ? mi : -INFINITY;
            mloc = fmaxf(mloc, li > 0.f ? mi : -INFINITY);
        }
        mloc = wave_max(mloc);
        if (lane == 0) sm_red[wid] = mloc;
        __syncthreads();
        M = fmaxf(fmaxf(sm_red[0], sm_red[1]), fmaxf(sm_red[2], sm_red[3]));
        __syncthreads();
        float lloc = 0.f;
        for (int i = tid; i < P.n_split; i += kAttnThreads) {
            const float wi = M == -INFINITY ? 0.f : fast_exp2(sm_w[i] - M);
            sm_w[i] = wi;
            lloc = fmaf(ld_agent(pml + 2 * i + 1), wi, lloc);
        }
        lloc = wave_sum(lloc);
        if (lane == 0) sm_red[wid] = lloc;
        __syncthreads();
        L = (sm_red[0] + sm_red[1]) + (sm_red[2] + sm_red[3]);
        o_t = 0.f;
        if (t < D) {
            const float* po = P.part_o + (size_t)bh * P.n_split * D + t;
            int i = 0;
            // 16 partial loads in flight before any is folded
            for (; i + 16 <= P.n_split; i += 16) {
                float x[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) x[u] = ld_agent(po + (size_t)(i + u) * D);
#pragma unroll
                for (int u = 0; u < 16; ++u) o_t = fmaf(x[u], sm_w[i + u], o_t);
            }
            for (; i < P.n_split; ++i) o_t = fmaf(ld_agent(po + (size_t)i * D), sm_w[i], o_t);
        }
        if (tid == 0)                            // ready for the next call
            __hip_atomic_store(&P.counters[pair], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // Join the new entry as a one-key partial: k_hat, v_hat are the rotated
    // key and the value rounded to the cache element type.
    const float* kv = P.k + (size_t)pair * D;
    const float* vv = P.v + (size_t)pair * D;
    S k_hat{}, v_hat{};
    float prod = 0.f;
    if (t < D) {
        const float kr = MODE == kModeStep ? rope_elem(kv, t, P.rot, P.log2_theta, p) : kv[t];
        k_hat = round_to_elt<DT>(kr);
        v_hat = round_to_elt<DT>(vv[t]);
        prod = sm_q[t] * elt_to_f32<DT>(k_hat);
    }
    prod = wave_sum(prod);
    if (lane == 0) sm_dot[wid] = prod;
    __syncthreads();
    const float s_new = (sm_dot[0] + sm_dot[1]) + (sm_dot[2] + sm_dot[3]);
    const float M2 = fmaxf(M, s_new);
    const float a = fast_exp2(M - M2);
    const float bn = fast_exp2(s_new - M2);
    const float L2 = fmaf(L, a, bn);
    if (t < D) {
        float o = fmaf(o_t, a, bn * elt_to_f32<DT>(v_hat)) / L2;
        if (MODE == kModeStep && P.gate != nullptr) o *= 1.f / (1.f + expf(-P.gate[bh]));
        P.out[(size_t)bh * D + t] = o;
    }

    if (MODE == kModeStep) {
        // Every split of this pair has finished reading (single split: the
        // barrier above; several: the arrival count), so the ring slot that
        // still held position p - S can be overwritten now.
        int row = -1;
        if (p >= 0) {
            if (RING) row = p % P.S;
            else if (p < P.S) row = p;
        }
        if (row < 0 && tid == 0 && g == 0 && p >= 0) atomicOr(P.err, 1);
        if (row >= 0 && t < D) {
            S* kd = reinterpret_cast<S*>(P.kc) + ((size_t)pair * P.S + row) * D;
            S* vd = reinterpret_cast<S*>(P.vc) + ((size_t)pair * P.S + row) * D;
            kd[t] = k_hat;
            vd[t] = v_hat;
        }
    }
}

}  // namespace hswd
