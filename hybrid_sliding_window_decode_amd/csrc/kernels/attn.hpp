// Decode attention over a ring or an append KV cache, with the new entry
// joined in score space, RoPE of the query in the prologue and, in the fused
// layer step, the head gate and the entry write in the epilogue.
//
// Summation order.  The valid key range of each (stream, kv head) is cut into
// chunks of K keys (K = keys_per_split; by default a ring's from its slot
// count, 128 to 512, and an append cache stream's from its own position, at
// most 1024 keys below 131072, 2048 below 524288 and from there 1024 per kv
// head within [2048, 8192], longer only past 4096 chunks).  A chunk's partial (max m, sum l, unnormalised o) is computed the
// same way wherever it runs: the workgroup's waves take the chunk's tiles
// round robin, keep an online softmax each, and merge through LDS in wave
// order.  Chunk partials are then
// folded in chunk order, and the new entry last.  The bits therefore depend
// on K and the positions only -- not on the batch, nor on how many chunks a
// workgroup streams, which the host picks from the batch and the CU count.
//
// Streaming.  One workgroup (4 waves) streams a contiguous range of chunks of
// one (stream, kv head).  Each wave reads whole 32-key (fp8), 16-key
// (bf16/f16) or 8-key (f32) tiles (at 256 dims) with 128-bit non-temporal
// loads, lanes over head dims, and keeps the next tile in flight while it
// scores the current one (register double buffering); the prefetch runs
// across chunk boundaries, and each wave's chunk partial goes to LDS, so the
// waves of the one-head kernel meet at a barrier only every four chunks.
// The grouped kernels for 4 and 8 query heads per kv head run both products
// on the matrix cores, staging K and then V through the wave's LDS rows.  The per-stream inputs and the first
// two tiles are requested before the prologue (RoPE of the query and the new
// key, the new entry's score).  Dot products are reduced across lanes with a
// transposed butterfly (about one exchange per key); every exchange is a DPP
// move or a gfx950 permlane swap, none goes through LDS.  Softmax is in base
// 2 with log2(e) folded into the query scale.
//
// Several workgroups per (stream, kv head) (long contexts, small batches):
// each stores its chunk partials with agent-scope atomic stores, counts its
// arrival, and the last to arrive folds all chunk partials (32 loads in
// flight before folding), joins the new entry, gates, and writes the entry
// into the cache -- after every read of that cache block, which the ring
// needs (its slot pos mod n_slots still holds position pos - n_slots, inside
// the window).
//
// Sources: vLLM-Omni fork commit log, score-space join commit (join scores,
// not keys; ring without reordering, only a mask; 511 slots) and Spark-X2.5
// model commit (per-type RoPE, sigmoid head gate); TensorFold pull request
// 608 review thread (split the key range to fill the GPU, merge partials,
// keep tiles in flight, issue the merge's loads before folding, the split
// size is part of the summation order); pega-omni pull request 4 (RoPE, ring
// write and attention in one launch; window loads issued before the sync on
// the rotated query).
#pragma once

#include "common.hpp"

#include <utility>

namespace hswd {

#ifndef HSWD_ATTN_WAVES
#define HSWD_ATTN_WAVES 4
#endif
constexpr int kAttnWaves = HSWD_ATTN_WAVES;          // waves per workgroup
constexpr int kAttnThreads = kAttnWaves * kWave;
static_assert(kAttnWaves == 4 || kAttnWaves == 8, "one thread per head dim needs >= 256 threads");
constexpr int kMaxChunks = 4096;                     // chunks per (stream, kv head)
constexpr int kAutoChunkKeys = 1024;                 // cap of a stream's own default chunk
constexpr int kAutoLongKeys = 1 << 17;               // ... doubled from this many keys on
constexpr int kAutoVeryLongKeys = 1 << 19;           // ... and 8x from this many keys on

// The cap from kAutoVeryLongKeys keys on: kAutoChunkKeys per kv head, 2 to
// 8 of them (a power of two), so that a lone stream there still has at
// least 512 chunks over its kv heads (one compute unit streams too little
// of the GPU's bandwidth for fewer workgroups to keep it busy), or as many
// as below that tier (fewer than 4 kv heads).
__host__ __device__ inline int auto_very_long_cap(int hkv) {
    return (hkv >= 8 ? 8 : hkv >= 4 ? 4 : 2) * kAutoChunkKeys;
}

// A stream's default chunk over an append cache, from its n valid keys: the
// smallest power of two >= n / 32, at least `floor` (four quanta, eight for
// grouped heads), at most kAutoChunkKeys below kAutoLongKeys keys, twice
// that below kAutoVeryLongKeys and auto_very_long_cap(hkv) from there, then
// doubled while n would need more than kMaxChunks chunks.  Nondecreasing in
// n.
// About 32 chunks spread a stream far below its cache's capacity over many
// workgroups; the cap keeps the chunks of long streams fine enough that
// their workgroups get even shares (a workgroup streams ceil(chunks /
// workgroups) of them, and one compute unit's bandwidth sets how long the
// busiest takes), and is raised for the longest streams, whose partials the
// last workgroup to arrive folds in sequence (2^20 keys over 8 kv heads:
// 128 of them, not 512).  The host sizes the launch with the same function.
__host__ __device__ inline int auto_chunk_keys(int n, int floor, int hkv) {
    const int target = (n + 31) >> 5;
    const int cap = n < kAutoLongKeys       ? kAutoChunkKeys
                    : n < kAutoVeryLongKeys ? 2 * kAutoChunkKeys
                                            : auto_very_long_cap(hkv);
    int k = floor;
    while (k < target && k < cap) k <<= 1;
    while ((n + (long)k - 1) / k > kMaxChunks) k <<= 1;
    return k;
}

// What a launch of the attention kernel produces.
enum AttnMode : int {
    kModeAttend = 0,    // o = attention output before the gate (q, k already rotated)
    kModeStep = 1,      // whole layer step: rope, attend, gate, write the entry
    kModePartials = 2,  // chunk partials of the cached keys only (natural-log m)
};

struct AttnParams {
    float* out;              // [B,H,D]
    const float* q;          // [B,H,D]: rotated (attend) or raw (step)
    const float* k;          // [B,Hkv,D]: rotated (attend) or raw (step); unused for partials
    const float* v;          // [B,Hkv,D]
    const float* gate;       // [B,H] logits, or null
    const float* gx;         // [B,hidden] gate-projection input, or null
    const float* gw;         // [H,hidden] gate-projection weight (used when gx != null)
    int hidden;
    const float* kv_scale;   // fp8 caches: [2,Hkv] per-head scales (K then V), or null
    void* kc;                // cache [B,Hkv,S,D]
    void* vc;
    const int32_t* pos;      // [B]
    float* part_o;           // chunk partials [B*H][n_chunk][D]
    float* part_ml;          // [B*H][n_chunk][2]
    int32_t* counters;       // merge arrivals [B*Hkv][npiece], then entry arrivals [B*Hkv] (npiece > 1)
    int32_t* err;            // error word
    int B, H, Hkv, S;        // S: ring slots or append capacity
    int K;                   // keys per chunk
    int n_chunk;             // chunks per (stream, kv head)
    int cpw;                 // chunks per workgroup
    int wpp;                 // workgroups per (stream, kv head)
    int ring;
    int max_pos;             // append: host bound of pos (grid size)
    int rot;
    double log2_theta;
    float qscale;            // softmax scale * log2(e)
    // 4- and 8-head kernels only: query heads per kv head in memory (H /
    // Hkv), and the pieces of G heads the launch splits each group into (a
    // group larger than G; 1 otherwise).  Every piece reads the cache; the
    // last to finish writes the new entry.
    int Gq, npiece;
    // append caches under the default chunking (auto_k 1, or 2 when the
    // caller fixed the chunks per workgroup): each stream's chunk is
    // auto_chunk_keys(its valid keys, k_floor), and K / cpw above are the
    // values of a stream at max_pos
    int auto_k, k_floor;
    // packed split (long append caches, default chunking, one piece per
    // group): the workgroups the launch deals out to the streams in
    // proportion to their valid keys, or 0 (the grid is pack + B * Hkv)
    int pack;
};

// Matrix-core kernels: 4 or 8 query heads per kv head over a 16-bit or fp8
// cache.  The score product is then a [G x D] . [D x keys] contraction (fp8
// keys become bf16, which holds every e4m3 value exactly) and the value
// product a [D x keys] . [keys x G] one (fp8 values become fp16, exact too).
template <int DT, int G>
constexpr bool use_mfma() {
    return (G == 4 || G == 8) && (DT == kBF16 || DT == kF16 || DT == kFP8);
}

// Tile geometry.  G query heads per kv head keep G query vectors and G
// accumulators per lane, so a grouped VALU kernel reads fp8 rows 8 bytes per
// lane (8 dims, as for 16-bit rows) and halves its 16-bit tiles (4 loads of
// K and of V instead of 8) to stay within 256 VGPRs (2 waves per SIMD);
// its fp8 tiles keep 8 loads, so a wave keeps as many bytes in flight as
// with 16-bit rows.  The MFMA kernels keep no query vectors in registers
// and keep 8-load tiles of 16 bytes per lane (fp8: 32 keys at 256 dims).
template <int D, int DT, int G = 1>
struct AttnGeo {
    static constexpr int EB = elt_bytes<DT>();        // element bytes
    static constexpr int CB = DT == kFP8 && G > 1 && !use_mfma<DT, G>() ? 8 : 16;   // bytes per lane chunk
    static constexpr int EPC = CB / EB;               // elements per chunk
    static constexpr int LPR = D / EPC;               // lanes per cache row
    static constexpr int RPI = kWave / LPR;           // rows per wave-wide load
    static constexpr int NL = G == 1 || use_mfma<DT, G>() || (G == 2 && DT == kFP8) ? 8 : 4;   // loads per tile
    static constexpr int KT = NL * RPI;               // keys per wave tile
    static constexpr int STEP = LPR / NL;             // lane stride between reduced keys
    static_assert(LPR >= NL && LPR <= kWave && kWave % LPR == 0, "geometry");
};

// Keys per chunk must be a multiple of this: a whole 8-load tile for every
// wave (the grouped kernels' 4-load tiles divide it).
constexpr int chunk_quantum(int D, int DT) {
    return kAttnWaves * 8 * (kWave / (D / (16 / (DT == kF32 ? 4 : (DT == kFP8 ? 1 : 2)))));
}

// Calls f(integral_constant<int, I>) for I = 0 .. N - 1, so each call can
// pass I on as an immediate operand.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The 16-block 4x4x4 matrix product with block AB's A operand broadcast to
// all 16 blocks (cbsz 4, abid AB): D[b][v][c] += sum_k A_AB[v][k] B_b[k][c],
// where lane 4 b + i holds A_b[i][0..3] and B_b[0..3][i], and register v of
// lane 4 b + c holds D[b][v][c] (layouts checked on the GPU with a probe
// before use).  BF: bf16 operands, else fp16.
typedef float f32x4v __attribute__((ext_vector_type(4)));
template <int AB, bool BF>
__device__ __forceinline__ f32x4v mfma4_bcast(const u32x2& a, const u32x2& b, const f32x4v& c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 4, AB, 0);
    else
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h16x4, a),
                                                 __builtin_bit_cast(h16x4, b), c, 4, AB, 0);
}

// Max of N values in LDS.
template <int N>
__device__ __forceinline__ float lds_max(const float* a) {
    float m = a[0];
#pragma unroll
    for (int i = 1; i < N; ++i) m = fmaxf(m, a[i]);
    return m;
}

// Fold partial (m, l, o) into the running (M, L, O); base-2 exponents.  The
// same arithmetic wherever it runs, so the order of folds fixes the bits.
// Empty partials (l == 0) are skipped; the first non-empty one is copied.
struct Fold {
    float M = -INFINITY, L = 0.f, O = 0.f;
    __device__ __forceinline__ void add(float m, float l, float o) {
        if (!(l > 0.f)) return;
        if (!(L > 0.f)) { M = m; L = l; O = o; return; }
        const float Mn = fmaxf(M, m);
        const float a = fast_exp2(M - Mn);
        const float b = fast_exp2(m - Mn);
        L = fmaf(L, a, l * b);
        O = fmaf(O, a, o * b);
        M = Mn;
    }
    // The same as add, with selects instead of branches (so a caller's
    // loads for several folds need not wait for one another).
    __device__ __forceinline__ void add_sel(float m, float l, float o) {
        const bool take = l > 0.f, have = L > 0.f;
        const float Mn = fmaxf(M, m);
        const float a = fast_exp2(M - Mn);
        const float b = fast_exp2(m - Mn);
        const float Lm = fmaf(L, a, l * b);
        const float Om = fmaf(O, a, o * b);
        M = take ? (have ? Mn : m) : M;
        L = take ? (have ? Lm : l) : L;
        O = take ? (have ? Om : o) : O;
    }
};

// Fold::add for E values sharing one (M, L): a partial (m, l, o[0..E)) into
// the running (M, L, O[0..E)), each O[e] exactly as Fold::add would fold
// it (M and L do not depend on O).
template <int E>
__device__ __forceinline__ void fold_row(float& M, float& L, float (&O)[E], float m, float l,
                                         const float (&o)[E]) {
    const bool take = l > 0.f, have = L > 0.f;
    const float Mn = fmaxf(M, m);
    const float a = fast_exp2(M - Mn);
    const float b = fast_exp2(m - Mn);
    const float Lm = fmaf(L, a, l * b);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float Om = fmaf(O[e], a, o[e] * b);
        O[e] = take ? (have ? Om : o[e]) : O[e];
    }
    M = take ? (have ? Mn : m) : M;
    L = take ? (have ? Lm : l) : L;
}

// One exchange of the transposed butterfly: a lane whose `M` bit is set
// ends with the sum over both lanes of the pair of the upper value, its
// partner with that of the lower one (each lane adds its own value first).
//   M = 16, 32: one permlane swap of (lo, hi) hands each lane exactly the
//               two addends it needs;
//   M = 4, 8:   both pair sums in DPP, then a select;
//   M = 1, 2:   the lane sends the value its partner keeps.
template <int M>
__device__ __forceinline__ float tstage(float lo, float hi, bool up) {
    if constexpr (M == 16 || M == 32) {
        float r0, r1;
        lane_swap<M>(lo, hi, r0, r1);
        return up ? r1 + r0 : r0 + r1;          // own value first, as below
    } else if constexpr (M == 8) {
        const float a = lo + dpp::mov<dpp::kRowRor8>(lo);
        const float b = hi + dpp::mov<dpp::kRowRor8>(hi);
        return up ? b : a;
    } else if constexpr (M == 4) {
        const float a = lo + dpp::mov<dpp::kRowShl4>(lo);   // lanes with bit 2 clear
        const float b = hi + dpp::mov<dpp::kRowShr4>(hi);   // lanes with bit 2 set
        return up ? b : a;
    } else {
        const float send = up ? lo : hi;
        const float keep = up ? hi : lo;
        return keep + xor_lane<M>(send);
    }
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
    for (int m = M3 / 2; m >= 1; m >>= 1) c = xor_sum_rt(c, m);
    return c;
}

// The same for four per-load partials: on exit this lane holds the full sum
// for load ((lane % LPR) / (LPR / 4)).
template <int LPR>
__device__ __forceinline__ float transposed_reduce4(const float (&v)[4], int lane) {
    constexpr int M1 = LPR / 2, M2 = LPR / 4;
    bool u = (lane & M1) != 0;
    const float a0 = tstage<M1>(v[0], v[2], u), a1 = tstage<M1>(v[1], v[3], u);
    u = (lane & M2) != 0;
    float c = tstage<M2>(a0, a1, u);
#pragma unroll
    for (int m = M2 / 2; m >= 1; m >>= 1) c = xor_sum_rt(c, m);
    return c;
}

// Chunk-partial slots per flush buffer: the LDS stash holds kStash chunks
// of every query head of the group, 32 KiB in all at 256 dims (the 8-head
// kernel's one slot sits over its waves' K / V rows instead).
template <int G>
constexpr int stash_slots() { return G == 1 ? 4 : (G == 2 ? 2 : 1); }

// Flush buffers of the wave chunk partials: two, used alternately, so a
// slot is rewritten only after the barrier of the flush in between; the
// 8-head kernel keeps one (its partials sit over the waves' K / V rows)
// and ends each flush with a second barrier instead.
template <int G>
constexpr int flush_buffers() { return G == 8 ? 1 : 2; }

// Totals over the workgroup's threads in one exchange: the 64-bit sum of
// w, and the maxima of a, b and c, floats that hold integers exactly (wave
// butterflies, then the waves' results meet in red: two sets of kAttnWaves
// x 4 slots, used alternately by successive calls, so one barrier per call
// suffices).  Exact, so every order gives the same totals.
__device__ __forceinline__ void deal_totals(long long (*red)[kAttnWaves][4], int& parity, int tid,
                                            long long& w, float& a, float& b, float& c) {
    for (int m = 1; m < kWave; m <<= 1) w += __shfl_xor(w, m, kWave);
    a = wave_max(a);
    b = wave_max(b);
    c = wave_max(c);
    long long(*r)[4] = red[parity];
    parity ^= 1;
    if (tid % kWave == 0) {
        r[tid / kWave][0] = w;
        r[tid / kWave][1] = __float_as_int(a);
        r[tid / kWave][2] = __float_as_int(b);
        r[tid / kWave][3] = __float_as_int(c);
    }
    __syncthreads();
    w = r[0][0];
    a = __int_as_float((int)r[0][1]), b = __int_as_float((int)r[0][2]),
    c = __int_as_float((int)r[0][3]);
    for (int v = 1; v < kAttnWaves; ++v) {
        w += r[v][0];
        a = fmaxf(a, __int_as_float((int)r[v][1]));
        b = fmaxf(b, __int_as_float((int)r[v][2]));
        c = fmaxf(c, __int_as_float((int)r[v][3]));
    }
}

// The sum alone, of integers below 2^24 held as floats (exact in any
// order), through the same exchange.
__device__ __forceinline__ float deal_sum(long long (*red)[kAttnWaves][4], int& parity, int tid,
                                          float v) {
    v = wave_sum(v);
    float* r = reinterpret_cast<float*>(red[parity]);
    parity ^= 1;
    if (tid % kWave == 0) r[tid / kWave] = v;
    __syncthreads();
    v = r[0];
    for (int w = 1; w < kAttnWaves; ++w) v += r[w];
    return v;
}

// The packed split's deal (see the kernel): every thread takes stream tid
// (tid < B).  A stream of nb chunks of K keys that gets c chunks per
// workgroup takes ceil(nb / c) workgroups, each streaming at most c * K
// keys; the deal is the smallest such bound M (a multiple of the smallest
// chunk, c = M / K for every stream) whose workgroups, Hkv per stream and
// workgroup slot, fit in the pack (every stream takes at least one; past
// pack / Hkv streams, in the launch's pack + B * Hkv), found by bisection
// between the balanced share of all chunks and the largest stream; then c
// is evened out over the stream's workgroups.  The thread whose stream owns
// workgroup w writes its role to role[0..4] (pair, workgroup of the pair,
// workgroups of the pair, chunks per workgroup, keys per chunk); role[0]
// stays -1 past the last stream's workgroups.  scan: 4 * kAttnThreads ints
// of LDS.  Not inlined: it runs once per launch, and its temporaries stay
// out of the kernel's register budget.
__device__ __attribute__((noinline)) void pack_deal(const int32_t* pos, int B, int Hkv, int S,
                                                    int max_pos, int k_floor, int pack, int w,
                                                    int tid, int* scan, int* role) {
    auto red = reinterpret_cast<long long(*)[kAttnWaves][4]>(scan);
    int* wsum = scan + 2 * kAttnWaves * 4 * 2;      // kAttnWaves ints past red
    int parity = 0;
    const int i = tid;                              // this thread's stream
    int nv_i = 0;
    if (i < B) {
        const int p_i = pos[i];
        nv_i = p_i < 0 ? 0 : (p_i < S ? p_i : S);
        if (nv_i > max_pos) nv_i = max_pos;
    }
    const int K_i = auto_chunk_keys(nv_i, k_floor, Hkv);
    const int nb_i = (nv_i + K_i - 1) / K_i;
    const long long keys_i = (long long)nb_i * K_i;  // keys of its chunks
    if (tid == 0) role[0] = -1;
    // all chunks' keys; the largest chunk, the smallest (as the largest
    // -K), the largest stream: powers of two and nb * K (nb < 2^24), exact
    // as floats
    long long W = keys_i;
    float fKmax = nb_i > 0 ? (float)K_i : 0.f, fKmin = nb_i > 0 ? -(float)K_i : -0x1p31f,
          fHi = (float)keys_i;
    deal_totals(red, parity, tid, W, fKmax, fKmin, fHi);
    // workgroups per kv head: the pack's, or with more streams than that
    // (no deal then fits the GPU at once) the launch's pack + B
    const int budget = B <= pack / Hkv ? pack / Hkv : pack / Hkv + B;
    int c_i = nb_i;                                 // chunks per workgroup (one workgroup)
    if (W > 0) {
        const unsigned Kmax = (unsigned)fKmax, Kmin = (unsigned)-fKmin, Hi = (unsigned)fHi;
        // bound M = m * Kmin, from lo: the balanced share (or the largest
        // chunk); at hi one workgroup per stream (B of them) fits.  32-bit
        // from here: Hi < 2^32, chunk sizes are powers of two, so c = m *
        // Kmin / K is a shift of m, and the counts stay below 2^24
        // (B * kMaxChunks).  W / (budget * Kmin) is exact enough in double
        // (W < 2^41) for its ceiling.
        const unsigned lo = max((unsigned)ceil((double)W / ((double)budget * Kmin)),
                                (Kmax + Kmin - 1) / Kmin);
        const unsigned hi = max(lo, (unsigned)(((unsigned long long)Hi + Kmin - 1) / Kmin));
        const int sh = nb_i > 0 ? __builtin_ctz((unsigned)K_i / Kmin) : 0;
        auto fits = [&](unsigned m) {
            unsigned n = 0;
            if (i < B) {
                const unsigned c = m >> sh;
                n = nb_i > 0 ? ((unsigned)nb_i + c - 1) / c : 1;
            }
            return deal_sum(red, parity, tid, (float)n) <= (float)budget;
        };
        // the smallest m that fits: lo itself (balanced streams), else
        // steps of 1, 2, 4, ... above it, then bisection of the last step
        unsigned good = hi, bad = lo;
        if (fits(lo)) {
            good = lo;
        } else {
            for (unsigned step = 1; bad + step < good; step *= 2) {
                if (fits(bad + step)) {
                    good = bad + step;
                    break;
                }
                bad += step;
            }
            while (good - bad > 1) {
                const unsigned mid = bad + (good - bad) / 2;
                if (fits(mid)) good = mid;
                else bad = mid;
            }
        }
        if (nb_i > 0) c_i = (int)min((unsigned)nb_i, good >> sh);
    }
    int w_i = 1, cw_i = 1;
    if (nb_i > 0) {
        w_i = (nb_i + c_i - 1) / c_i;
        cw_i = (nb_i + w_i - 1) / w_i;              // even shares, same count
        w_i = (nb_i + cw_i - 1) / cw_i;
    }
    // this stream's first workgroup: exclusive prefix of Hkv * w over the
    // streams (wave scans, then the waves' totals)
    const int c_own = i < B ? w_i * Hkv : 0;
    int incl = c_own;
    for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off, kWave);
        if (tid % kWave >= off) incl += v;
    }
    if (tid % kWave == kWave - 1) wsum[tid / kWave] = incl;
    __syncthreads();
    for (int v = 0; v < tid / kWave; ++v) incl += wsum[v];
    const int excl = incl - c_own;
    if (i < B && w >= excl && w < incl) {
        const int li = w - excl;
        role[0] = i * Hkv + li % Hkv;
        role[1] = li / Hkv;
        role[2] = w_i;
        role[3] = cw_i;
        role[4] = K_i;
    }
}

// G = H / Hkv query heads share each kv head (grouped-query attention by
// reshaping the query, the talker commit): one workgroup scores all G of
// them against every K/V tile it loads, so the cache is read once per group.
// Two workgroups of 4 waves per CU (2 waves per SIMD): at most 256 VGPRs.
// SHARED: a group larger than G is split into pieces of G heads whose
// workgroups read the same rows at about the same time (plain loads).
template <int D, int DT, bool RING, int MODE, int G, bool SHARED>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_kernel(AttnParams P) {
    using Geo = AttnGeo<D, DT, G>;
    using S = typename Storage<DT>::type;
    constexpr int EPC = Geo::EPC, LPR = Geo::LPR, RPI = Geo::RPI, NL = Geo::NL, KT = Geo::KT;
    constexpr float kLn2 = 0.69314718055994531f;
    constexpr int kStash = stash_slots<G>();
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "query heads per kv head");
    static_assert(G != 8 || use_mfma<DT, G>(), "8 query heads per kv head: matrix-core kernel");
    constexpr int NB = flush_buffers<G>();

    constexpr bool MF = use_mfma<DT, G>();
    // The matrix-core kernels take the value product on the matrix cores
    // too: V goes through the wave's LDS rows after its K, the probabilities
    // stay in the registers the score product left them in, and the product
    // is a series of 16-block 4x4x4 products, each with the probabilities of
    // 4 keys for 4 heads broadcast to all 16 blocks (4 dims each): a lane
    // accumulates 4 heads of one dim per 64 dims, D / 16 registers per set of
    // 4 heads.  Two V tiles in flight for 16-bit caches at 128 dims, one
    // otherwise (VS1: V of the next tile requested once this tile's is in
    // LDS).
    // fp8 caches (F8): 32-key tiles at 256 dims (64 at 128), K and V staged
    // in LDS as the fp8 codes they are and converted as they are read back
    constexpr bool F8 = MF && DT == kFP8;
    constexpr int NQ = G / 4;                 // sets of 4 heads (matrix-core kernels)
    constexpr bool VS1 = MF && (D == 256 || F8);
    // 8-head kernel (OA): each wave writes its chunk partial (8 heads x D
    // floats) over its own K / V rows, free at a chunk end, so the partials
    // take no LDS of their own (two workgroups per CU); every flush ends
    // with a barrier before any wave stages its next tile there
    constexpr bool OA = MF && G == 8;
    static_assert(!OA || NB == 1, "partials over the K / V rows: one flush buffer");
    // fp16 probabilities of the matrix-core kernels over f16 / fp8 caches
    // are scaled by 2^kPScale; a wave's chunk partial (sum and values) is
    // scaled back by kPUnscale, a power of two, when the chunk ends
    constexpr float kPScale = MF && DT != kBF16 ? 15.f : 0.f;
    constexpr float kPUnscale = MF && DT != kBF16 ? 0x1p-15f : 1.f;
    // MFMA kernel: each wave stages its K rows (then its V rows) in LDS
    // (rows padded by 16 bytes so the 16 rows an operand read touches fall
    // in distinct banks; fp8 keys as exact bf16, fp8 values as exact fp16),
    // and the query heads sit there as 16-bit hi + lo parts.
    constexpr int KPAD = D * 2 / 16 + 1;                  // 16-byte units per staged (16-bit) row
    // V rows are staged 32 bytes apart instead (VPAD)
    constexpr int VPAD = D * 2 / 16 + 2;
    // F8 rows: D code bytes plus 16, so the 16 rows of a score-operand read
    // fall in distinct banks
    constexpr int P8 = D / 16 + 1;                        // 16-byte units per staged fp8 row
    __shared__ float sm_q[MF ? 1 : G][D];
    __shared__ u32x4 sm_k[MF ? kAttnWaves : 1][MF ? KT * (F8 ? P8 : VPAD) : 1];   // K rows, then V rows
    static_assert(!OA || G * D * 4 <= KT * (F8 ? P8 : VPAD) * 16, "a wave's partial fits its K / V rows");
    // query rows padded by 16 bytes too: unpadded, the G heads' rows (512
    // bytes apart) would share banks and the operand reads conflict 4 ways
    __shared__ __attribute__((aligned(16))) uint16_t sm_qh[MF ? G + 1 : 1][MF ? D + 8 : 1];
    __shared__ __attribute__((aligned(16))) uint16_t sm_ql[MF ? G + 1 : 1][MF ? D + 8 : 1];
    // (both read 16 bytes at a time: aligned to 16)
    // wave chunk partials, by flush parity (8-head kernel: over the K / V rows)
    __shared__ __attribute__((aligned(16))) float sm_o[OA ? 1 : NB][OA ? 1 : kStash][OA ? 1 : G][OA ? 1 : kAttnWaves][OA ? 1 : D];
    __shared__ float sm_m[NB][kStash][G][kAttnWaves], sm_l[NB][kStash][G][kAttnWaves];
    __shared__ float sm_dot[G][kAttnWaves];
    __shared__ float sm_gl[G][kAttnWaves];
    __shared__ int sm_last;
    // MFMA kernel: the running fold of the chunk partials (single workgroup
    // per pair) lives in LDS, not registers (it is touched once per chunk),
    // head-major like the flush: M and L per head (the head's first flush
    // thread stores them; the head's threads, all in one wave, read them
    // back), O per (head, dim).
    __shared__ float sm_run_ml[MF ? G : 1][2];
    __shared__ float sm_run_o[MF ? G : 1][MF ? D : 1];
    __shared__ float sm_glogit[MF ? G : 1];       // MFMA kernel: the given gate logits
    __shared__ float sm_vh[MF ? D : 1];           // MFMA kernel: the new entry's value

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // (the matrix-core kernels take the wave index as a scalar; the VALU
    // kernels measure 1-2% faster with it in a vector register)
    const int wid = use_mfma<DT, G>() ? __builtin_amdgcn_readfirstlane(tid / kWave) : tid / kWave;
    const int t = tid;                                 // this thread's head dim (t < D)

    // Workgroup -> (stream, kv head, head piece, chunk range).  When the
    // pair count allows, the workgroups of one pair go to the same XCD
    // (workgroups are dealt to the 8 XCDs round robin) and are dealt out
    // together: the merging one finds the partials in its L2, and the pieces
    // of a large group, which read the same K/V rows at about the same
    // time, share them there.
    const int n_pairs = P.B * P.Hkv;
    const int npiece = G >= 4 ? P.npiece : 1;
    const int per_pair = npiece * P.wpp;
    int pair, sub;
    // Packed split: every workgroup reads all positions and deals at most
    // P.pack workgroups out to the streams (the fewest keys per workgroup
    // that fit; at least one workgroup each, at most one per chunk of the
    // stream's own size), in stream order, Hkv consecutive workgroups (one
    // per kv head) per round of a stream; workgroups past the last
    // stream's exit at once.  Only the work split follows from it, never a
    // stream's chunks or their order.  The same integer arithmetic in every
    // workgroup gives every workgroup the same deal.
    const bool packed = !RING && MODE != kModePartials && P.pack > 0 && npiece == 1;
    int pack_parts = 0, pack_cw = 0, pack_K = 0;
    if (packed) {
        // scratch for the scans: LDS no other code touches before the tiles
        int* scan = MF ? reinterpret_cast<int*>(&sm_k[0][0]) : reinterpret_cast<int*>(&sm_o[0][0][0][0][0]);
        int* role = scan + 4 * kAttnThreads + 8;
        pack_deal(P.pos, P.B, P.Hkv, P.S, P.max_pos, P.k_floor, P.pack, (int)blockIdx.x, tid,
                  scan, role);
        __syncthreads();
        // (uniform values: held in scalar registers)
        pair = __builtin_amdgcn_readfirstlane(role[0]);
        if (pair < 0) return;                           // past the last stream's workgroups
        sub = __builtin_amdgcn_readfirstlane(role[1]);
        pack_parts = __builtin_amdgcn_readfirstlane(role[2]);
        pack_cw = __builtin_amdgcn_readfirstlane(role[3]);
        pack_K = __builtin_amdgcn_readfirstlane(role[4]);
        __syncthreads();                                // the scratch is free again
    } else {
        const int w = blockIdx.x;
        if ((n_pairs & 7) == 0 && per_pair > 1) {
            const int k = w >> 3;
            pair = (k / per_pair) * 8 + (w & 7);
            sub = k % per_pair;
        } else {
            pair = w / per_pair;
            sub = w % per_pair;
        }
    }
    const int piece = packed ? 0 : sub / P.wpp;
    const int wg = packed ? sub : sub % P.wpp;
    const int b = pair / P.Hkv;
    const int g = pair % P.Hkv;
    // query heads of this workgroup: bh0 .. bh0 + gv - 1 (the 4- and 8-head
    // kernels can cover a piece of a larger group, or a smaller group with
    // heads idle)
    const int gv = G >= 4 ? min(G, P.Gq - piece * G) : G;
    const int bh0 = b * P.H + (G >= 4 ? g * P.Gq + piece * G : g * G);
    const float kscale = DT == kFP8 && P.kv_scale != nullptr ? P.kv_scale[g] : 1.f;
    const float vscale = DT == kFP8 && P.kv_scale != nullptr ? P.kv_scale[P.Hkv + g] : 1.f;
    // Chunk size and chunks per workgroup: the launch's (P.K, P.cpw), or
    // for an append cache under the default chunking the stream's own, set
    // once its position arrives (until then the first tiles are requested
    // on the launch's values, which the streams at the longest position
    // share).
    int K = packed ? pack_K : P.K, cpw = packed ? pack_cw : P.cpw;
    int c_begin = wg * cpw;
    int c_end = min(c_begin + cpw, P.n_chunk);
    int TPW = K / (KT * kAttnWaves);                  // tiles per wave in a full chunk

    const int c = lane % LPR;       // 16-byte chunk of the row this lane reads
    const int r = lane / LPR;       // row within a wave-wide load
    float qs[G][EPC];               // this lane's query dims, set after the prologue
    // matrix-core kernels: the query's MFMA operands (hi and lo, D / 32
    // slices), in registers for the whole launch (set after the prologue)
    u32x4 qhr[MF ? D / 32 : 1], qlr[MF ? D / 32 : 1];

    // This pair's K and V blocks: as lane pointers (VALU kernels), and as
    // the uniform block base plus a 32-bit lane offset (matrix-core kernels,
    // 2-8% faster there; the host caps a block at 4 GiB).  Each form is the
    // faster one for its kernels.
    constexpr int ROWB = D * Geo::EB;
    const S* kbase = reinterpret_cast<const S*>(P.kc) + (size_t)pair * P.S * D + c * EPC;
    const S* vbase = reinterpret_cast<const S*>(P.vc) + (size_t)pair * P.S * D + c * EPC;
    const char* kblk = reinterpret_cast<const char*>(P.kc) + (size_t)pair * P.S * ROWB;
    const char* vblk = reinterpret_cast<const char*>(P.vc) + (size_t)pair * P.S * ROWB;
    const uint32_t lane_col = (uint32_t)(c * Geo::CB);

    float m_run[G], l_lane[G], o_acc[G][EPC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m_run[hh] = -INFINITY;
        l_lane[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) o_acc[hh][e] = 0.f;
    }
    // MFMA kernel: the running max and sum of head (lane % 16) over the keys
    // this lane's group of 4 holds; lanes of heads >= G carry unused values
    float m1 = -INFINITY, l1 = 0.f;
    // value product on the matrix cores: O (4 heads x 64 dims) per set z of
    // 4 heads and group m of 64 dims, pv_acc[z * D / 64 + m]; lane l holds
    // dim 64 m + l of heads 4 z + i, i = 0..3
    typedef float pv4 __attribute__((ext_vector_type(4)));
    constexpr int NACC = MF ? NQ * (D / 64) : 1;
    pv4 pv_acc[NACC];
#pragma unroll
    for (int m = 0; m < NACC; ++m) pv_acc[m] = pv4{0.f, 0.f, 0.f, 0.f};
    Fold run[G];                    // folded chunk partials (wpp == 1)

    using Chunk = typename ChunkT<Geo::CB>::type;
    Chunk kA[NL], vA[NL], kB[NL], vB[NL];
    // MFMA kernel: K goes to LDS as soon as it arrives, so one register tile
    // of K suffices (LDS is its second buffer); kA, kB are then unused.
    Chunk kR[MF ? NL : 1];

    // Item j of this wave: tile (wid + 4 i) of chunk c_begin + j / TPW for
    // the full chunks, tile (wid + 4 (j - n_full_items)) of the partly valid
    // chunk after them.  A chunk is TPW * 4 tiles long, so both give the
    // first key c_begin * K + (4 j + wid) * KT, with no division.  Rows at
    // or past nv (only in the partly valid chunk, whose tiles end inside it,
    // or in a prefetch the loop never scores) are clamped onto row jlast =
    // nv - 1 (row 0 when nothing is valid), so every load stays inside this
    // (stream, kv head)'s written rows and may be issued unconditionally;
    // the softmax masks keys >= nv.  The first two tiles go out before the
    // position has arrived, clamped onto the block's last row S - 1 instead;
    // a wave whose first two tiles reach past nv requests them again once nv
    // is known (a stream with few keys), so no unwritten row is ever scored.
    int key0 = c_begin * K + wid * KT;
    int jlast = P.S - 1;
    auto item_key = [&](int j) __attribute__((always_inline)) { return key0 + j * (kAttnWaves * KT); };

    // Row `row` (already clamped onto jlast) of a block, matrix-core form.
    // (A uniform branch skipping the clamp where it changes nothing cost the
    // VALU kernels 1-4%.)
    auto blk_load = [&](const char* blk, int row) __attribute__((always_inline)) {
        return load_kv<Geo::CB, SHARED>(
            reinterpret_cast<const S*>(blk + ((uint32_t)row * ROWB + lane_col)));
    };

    auto load_k = [&](int j) __attribute__((always_inline)) {     // MFMA kernel only
        const int base = item_key(j) + r;
#pragma unroll
        for (int i = 0; i < (MF ? NL : 1); ++i) kR[i] = blk_load(kblk, min(base + i * RPI, jlast));
    };

    auto load_tile = [&](Chunk (&kt)[NL], Chunk (&vt)[NL], int j) __attribute__((always_inline)) {
        const int base = item_key(j) + r;
        if constexpr (!MF) {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int row = min(base + i * RPI, jlast);
                kt[i] = load_kv<Geo::CB, SHARED>(kbase + (size_t)row * D);
            }
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int row = min(base + i * RPI, jlast);
            if constexpr (MF) vt[i] = blk_load(vblk, row);
            else vt[i] = load_kv<Geo::CB, SHARED>(vbase + (size_t)row * D);
        }
    };

    // Per-stream inputs first: this thread's query dim and its RoPE partner
    // for every head of the group, and for the new entry the same of the key
    // plus the value (threads past D read dim 0 and drop it).  Vector loads
    // retire in order, so the prologue waits for these alone; the first two
    // tiles, requested next, stay in flight under its double-precision RoPE.
    // None of these waits for the stream's position, read only afterwards:
    // the first tiles' rows are clamped onto the block's last row.  Those two
    // requests are unconditional: a load under a branch would make the
    // compiler's wait counts at the join assume the branch was not taken, and
    // the prologue would wait for the tiles too.  (The one branch with loads,
    // the re-request of the first tiles of a stream with few keys, comes
    // after them: only its own, rare path waits longer.)
    const bool has_new = MODE != kModePartials;
    const int td = t < D ? t : 0;
    const bool rotated = MODE == kModeStep && td < P.rot;
    const int tp = MODE == kModeStep ? rope_partner(td, P.rot) : td;
    const float* qv = P.q + (size_t)bh0 * D;
    const float* kv = P.k + (size_t)pair * D;
    const float* vv = P.v + (size_t)pair * D;
    float q_t[G], q_p[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        q_t[hh] = hh < gv ? qv[(size_t)hh * D + td] : 0.f;      // idle heads: zero query
        q_p[hh] = hh < gv ? qv[(size_t)hh * D + tp] : 0.f;
    }
    float k_t = 0.f, k_p = 0.f, v_t = 0.f;
    if (has_new) {
        k_t = kv[td];
        k_p = kv[tp];
        v_t = vv[td];
    }
    const bool gproj = MODE == kModeStep && P.gx != nullptr;
    float glogit[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
        glogit[hh] = MODE == kModeStep && !gproj && P.gate != nullptr && hh < gv ? P.gate[bh0 + hh]
                                                                                 : 0.f;

    if constexpr (MF) load_k(0);
    load_tile(kA, vA, 0);
    if constexpr (!VS1) load_tile(kB, vB, 1);

    // The stream's position, requested after the first loads.
    const int p = P.pos[b];

    // Valid cache rows: ring slots s < min(p, S); append rows < p.
    int nv = p < 0 ? 0 : (p < P.S ? p : P.S);
    bool respread = false;
    if (!RING) {
        // keys at or past the launch's bound are not read (flagged)
        const int grid_keys = P.auto_k ? P.max_pos : P.n_chunk * K;
        if (nv > grid_keys) nv = grid_keys;
        if (MODE != kModePartials && wg == 0 && g == 0 && tid == 0 && p > P.max_pos)
            atomicOr(P.err, 2);
        if (P.auto_k && !packed) {
            // (packed split: already the stream's own, from the deal)
            // the stream's chunk (auto_chunk_keys), a function of its
            // position alone; its chunks spread over the pair's workgroups,
            // each taking at least the share of a stream at max_pos (the
            // launch's cpw): a shorter stream never needs to finish sooner
            // than the longest, and leaves compute units whose bandwidth the
            // longest streams' workgroups then have to themselves
            const int k = auto_chunk_keys(nv, P.k_floor, P.Hkv);
            const int nb = max(1, (nv + k - 1) / k);
            const int cw = P.auto_k == 2 ? cpw : max(cpw, (nb + P.wpp - 1) / P.wpp);   // 2: caller's split
            if (k != K || cw != cpw) {
                K = k;
                cpw = cw;
                c_begin = wg * cpw;
                c_end = min(c_begin + cpw, P.n_chunk);
                TPW = K / (KT * kAttnWaves);
                key0 = c_begin * K + wid * KT;
                respread = true;
            }
        }
        // the last workgroup of a pair also covers the grid's chunks past
        // the stream's own (empty partials for the partials entry)
        if (MODE == kModePartials && wg == P.wpp - 1) c_end = P.n_chunk;
    }
    if (MODE != kModePartials && wg == 0 && g == 0 && tid == 0 && p < 0) atomicOr(P.err, 4);

    // This workgroup's chunks [c_begin, c_end): full ones [c_begin, c_full),
    // then at most one partly valid chunk [c_full, c_valid); the rest hold no
    // valid key.
    const int n_valid_chunks = (nv + K - 1) / K;
    const int c_valid = max(c_begin, min(c_end, n_valid_chunks));
    const int c_full = max(c_begin, min(c_valid, nv / K));
    const int n_full_items = (c_full - c_begin) * TPW;
    // tiles of the partly valid chunk, per wave (the maximum over the waves,
    // so every wave runs the same loop; surplus tiles are fully masked)
    const int part_tiles = c_valid > c_full ? (nv - c_full * K + KT - 1) / KT : 0;
    const int part_items = (part_tiles + kAttnWaves - 1) / kAttnWaves;
    const int n_items = n_full_items + part_items;

    jlast = max(nv, 1) - 1;
    // the first two tiles reach past the valid rows, or the stream's chunks
    // start elsewhere than the launch's guess
    if (respread || item_key(1) + KT > nv) {
        if constexpr (MF) load_k(0);
        load_tile(kA, vA, 0);
        if constexpr (!VS1) load_tile(kB, vB, 1);
    }

    auto compute_tile = [&](const Chunk (&kt)[NL], const Chunk (&vt)[NL], int j) __attribute__((always_inline)) {
        const int jend = nv;
        const int tile0 = item_key(j);
        if constexpr (MF) {
            // Scores on the matrix cores.  The wave's K rows go to its LDS
            // rows (as loaded: row i * RPI + r, 16 bytes at chunk c) and come
            // back as MFMA operands: S^T[key][head] = K . Q^T for 16 keys at
            // a time (v_mfma_f32_16x16x32 over 32 dims per slice), with the
            // query in hi + lo 16-bit parts (about 16 significant bits) and
            // fp32 accumulation.  Lane l then holds keys 4 (l / 16) + i of
            // head l % 16; heads >= G read a zero query.
            using OpT = typename std::conditional<DT == kF16, _Float16, __bf16>::type;
            typedef OpT op8 __attribute__((ext_vector_type(8)));
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            constexpr int NG = KT / 16, NS = D / 32;
            const int hq = lane & 15, kq = lane >> 4;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                if constexpr (F8) sm_k[wid][(i * RPI + r) * P8 + c] = kR[i];
                else sm_k[wid][(i * RPI + r) * KPAD + c] = kR[i];
            }
            // the next item's K into the freed registers, in flight under
            // this tile's scores and values (rows clamped past the last item)
            load_k(j + 1);
            // four accumulators per key group (query hi / lo part, even / odd
            // slice) keep the matrix-core chains short; summed at the end
            f32x4 acc[NG][4];
#pragma unroll
            for (int kg = 0; kg < NG; ++kg) {
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[kg][u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // the query operands are in registers (qhr, qlr: read once per launch)
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                const u32x4& qh = qhr[sl];
                const u32x4& ql = qlr[sl];
#pragma unroll
                for (int kg = 0; kg < NG; ++kg) {
                    u32x4 a;
                    if constexpr (F8) {
                        // the 8 codes of dims 32 sl + 8 kq .. + 7, as exact bf16
                        const uint8_t* k8 = reinterpret_cast<const uint8_t*>(&sm_k[wid][(kg * 16 + hq) * P8]);
                        a = fp8x8_to_bf16x8(*reinterpret_cast<const u32x2*>(k8 + 32 * sl + 8 * kq));
                    } else {
                        a = sm_k[wid][(kg * 16 + hq) * KPAD + 4 * sl + kq];
                    }
                    f32x4& ah = acc[kg][2 * (sl & 1)];
                    f32x4& al_ = acc[kg][2 * (sl & 1) + 1];
                    if constexpr (DT != kF16) {
                        ah = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(op8, a), __builtin_bit_cast(op8, qh), ah, 0, 0, 0);
                        al_ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(op8, a), __builtin_bit_cast(op8, ql), al_, 0, 0, 0);
                    } else {
                        ah = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(op8, a), __builtin_bit_cast(op8, qh), ah, 0, 0, 0);
                        al_ = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(op8, a), __builtin_bit_cast(op8, ql), al_, 0, 0, 0);
                    }
                }
            }
            // online softmax per head over this lane's keys, the head's max
            // across its 4 lanes (distances 16 and 32)
            float sv[NG][4];
            float mx = -INFINITY;
#pragma unroll
            for (int kg = 0; kg < NG; ++kg) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = tile0 + kg * 16 + 4 * kq + i;
                    const float sc = (acc[kg][0][i] + acc[kg][1][i]) + (acc[kg][2][i] + acc[kg][3][i]);
                    sv[kg][i] = key < jend ? sc : -INFINITY;
                    mx = fmaxf(mx, sv[kg][i]);
                }
            }
            mx = xor_max<16>(mx);
            mx = xor_max<32>(mx);
            if (mx == -INFINITY) {                      // nothing valid in this tile
                if constexpr (VS1) load_tile(kA, vA, j + 1);
                return;
            }
            const float m_new = fmaxf(m1, mx);
            const float alpha = fast_exp2(m1 - m_new);
            m1 = m_new;
            // The probabilities are the A operand of P.V as they stand:
            // lane l holds keys 4 (l / 16) + i of head l % 16, so lanes
            // 16 s + 4 z .. + 3 hold the operand of block 4 s + z (rows:
            // heads 4 z .. 4 z + 3, k: keys 4 s + i).  f16 / fp8 caches: fp16 weights
            // (times 2^kPScale, undone at the chunk end), the running sum
            // over the same rounded values; bf16 caches: the weight as a
            // bf16 hi part plus a bf16 lo part (about 16 significant
            // bits), the running sum over the float weights.
            typedef short s16x4 __attribute__((ext_vector_type(4)));
            typedef int i32x2 __attribute__((ext_vector_type(2)));
            s16x4 pb[NG], pbl[NG];
            float psum = 0.f;
#pragma unroll
            for (int kg = 0; kg < NG; ++kg) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (DT != kBF16) {
                        const _Float16 ph = (_Float16)fast_exp2(sv[kg][i] - m_new + kPScale);
                        psum += (float)ph;
                        pb[kg][i] = __builtin_bit_cast(short, ph);
                    } else {
                        const float pr = fast_exp2(sv[kg][i] - m_new);
                        psum += pr;
                        const uint16_t hi = round_to_elt<kBF16>(pr);
                        pb[kg][i] = (short)hi;
                        pbl[kg][i] = (short)round_to_elt<kBF16>(pr - elt_to_f32<kBF16>(hi));
                    }
                }
            }
            l1 = l1 * alpha + psum;
            // rescale the accumulators (skipped when no head's max moved):
            // every lane holds heads 4 z .. 4 z + 3 of set z, whose factors
            // lanes 4 z .. 4 z + 3 hold
            if (__any(alpha != 1.f)) {
                const int ab = __builtin_bit_cast(int, alpha);
#pragma unroll
                for (int z = 0; z < NQ; ++z) {
                    const pv4 al4{__builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, 4 * z)),
                                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, 4 * z + 1)),
                                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, 4 * z + 2)),
                                  __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, 4 * z + 3))};
#pragma unroll
                    for (int m = 0; m < D / 64; ++m) pv_acc[z * (D / 64) + m] *= al4;
                }
            }
            // V to the wave's LDS rows, where its K was (this wave has
            // read them; its LDS accesses complete in order); fp8 codes as
            // they are
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                if constexpr (F8) sm_k[wid][(i * RPI + r) * P8 + c] = vt[i];
                else sm_k[wid][(i * RPI + r) * VPAD + c] = vt[i];
            }
            // one V tile in flight: the next one into the registers just
            // staged (rows clamped past the last item, as for K)
            if constexpr (VS1) load_tile(kA, vA, j + 1);
            {
                // per 4 keys, 64 dims and 4 heads one 16-block 4x4x4
                // product, O[head][dim] += P[head][key] V[key][dim], its A
                // operand (P: 4 heads x 4 keys) broadcast from the block
                // whose lanes hold those keys (lanes 16 s + 4 z .. + 3 hold
                // keys 4 s + i of heads 4 z .. 4 z + 3: block 4 s + z) and
                // its B operand V (4 keys x 4 dims per block), lane l
                // holding dim 64 m + l of the 4 keys.  The transposing LDS
                // reads give exactly that when every 16-lane group points at
                // the same keys, group q at dims 64 m + 16 q .. + 15.
                if constexpr (F8) {
                    // 8-bit read: lanes 2 j, 2 j + 1 of a group point at 8
                    // codes each of key 8 e + j; lane i receives code i of
                    // the 8 keys, in key order (fp16 in registers, exact)
                    const uint8_t* vb = reinterpret_cast<const uint8_t*>(&sm_k[wid][0]) +
                                        ((lane & 15) >> 1) * (P8 * 16) + 16 * kq + 8 * (lane & 1);
                    static_for<KT / 8>([&](auto ec) {
                        constexpr int e = decltype(ec)::value;
                        constexpr int n = e / 2, s0 = (2 * e) % 4;   // 16-key group, first 4-key block
                        const u32x2 pa = __builtin_bit_cast(u32x2, pb[n]);
#pragma unroll
                        for (int m = 0; m < D / 64; ++m) {
                            const u32x2 v8 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                (__attribute__((address_space(3))) i32x2*)(vb + 8 * e * (P8 * 16) + 64 * m)));
                            const u32x4 vh = fp8x8_to_f16x8(v8);
                            static_for<NQ>([&](auto zc) {
                                constexpr int z = decltype(zc)::value;
                                pv4& acc4 = pv_acc[z * (D / 64) + m];
                                acc4 = mfma4_bcast<4 * s0 + z, false>(pa, u32x2{vh.x, vh.y}, acc4);
                                acc4 = mfma4_bcast<4 * s0 + 4 + z, false>(pa, u32x2{vh.z, vh.w}, acc4);
                            });
                        }
                    });
                } else {
                    // 16-bit read: lanes 4 j .. 4 j + 3 of a group point at
                    // 4 dims each of key 4 s + j; lane i receives element i
                    // of the 4 keys
                    const uint16_t* vb = reinterpret_cast<const uint16_t*>(&sm_k[wid][0]) +
                                         ((lane & 15) >> 2) * (VPAD * 8) + 16 * kq + 4 * (lane & 3);
#pragma unroll
                    for (int kg = 0; kg < NG; ++kg) {
                        const u32x2 ph = __builtin_bit_cast(u32x2, pb[kg]);
                        static_for<4>([&](auto sc) {
                            constexpr int s4 = decltype(sc)::value;
                            const uint16_t* vrow = vb + (16 * kg + 4 * s4) * (VPAD * 8);
#pragma unroll
                            for (int m = 0; m < D / 64; ++m) {
                                const u32x2 va = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                    (__attribute__((address_space(3))) s16x4*)(vrow + 64 * m)));
                                static_for<NQ>([&](auto zc) {
                                    constexpr int z = decltype(zc)::value;
                                    pv4& acc4 = pv_acc[z * (D / 64) + m];
                                    acc4 = mfma4_bcast<4 * s4 + z, DT == kBF16>(ph, va, acc4);
                                    if constexpr (DT == kBF16)
                                        acc4 = mfma4_bcast<4 * s4 + z, true>(
                                            __builtin_bit_cast(u32x2, pbl[kg]), va, acc4);
                                });
                            }
                        });
                    }
                }
            }
        } else {
            float s[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float part[NL];
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    float kf[EPC];
                    unpack_chunk<DT>(kt[i], kf);
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc = fmaf(qs[hh][e], kf[e], acc);
                    part[i] = acc;
                }
                if constexpr (NL == 8) s[hh] = transposed_reduce8<LPR>(part, lane);
                else s[hh] = transposed_reduce4<LPR>(part, lane);
            }
            const int ki = (lane % LPR) / Geo::STEP;        // load index of this lane's key
            const int key = tile0 + ki * RPI + r;
            const bool valid = key < jend;
            // tile max over the distinct keys (lane bits >= STEP), per head
            float mx[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                s[hh] = valid ? s[hh] : -INFINITY;
                mx[hh] = s[hh];
#pragma unroll
                for (int m = Geo::STEP; m < kWave; m <<= 1) mx[hh] = xor_max_rt(mx[hh], m);
            }
            if (mx[0] == -INFINITY) return;                 // nothing valid in this tile
            float pr[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                const float m_new = fmaxf(m_run[hh], mx[hh]);
                const float alpha = fast_exp2(m_run[hh] - m_new);
                pr[hh] = fast_exp2(s[hh] - m_new);
                m_run[hh] = m_new;
                l_lane[hh] = l_lane[hh] * alpha + ((lane & (Geo::STEP - 1)) == 0 ? pr[hh] : 0.f);
#pragma unroll
                for (int e = 0; e < EPC; ++e) o_acc[hh][e] *= alpha;
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                // every key's probability to the lanes of its row, all requests
                // out before the first is used
                float pk[NL];
#pragma unroll
                for (int i = 0; i < NL; ++i) pk[i] = lane_value(pr[hh], r * LPR + i * Geo::STEP);
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    float vf[EPC];
                    unpack_chunk<DT>(vt[i], vf);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) o_acc[hh][e] = fmaf(pk[i], vf[e], o_acc[hh][e]);
                }
            }
        }
    };

    // End of a chunk (every wave, same point): the wave's partial for it
    // (reduced across lanes first in the one- and two-head kernels) is
    // written to its LDS slot of the current flush buffer.  Every kStash chunks, and once at the end, the buffer is
    // flushed: one barrier, then each thread forms the chunk partials for its
    // dim t, in chunk order, and folds (single workgroup per pair) or stores
    // them.  The two buffers alternate, so a slot is rewritten only after the
    // barrier of the flush in between; deferring the barrier keeps small
    // chunks cheap, and the arithmetic and its order are those of a barrier
    // per chunk.
    int n_st = 0, st_first = 0, n_flush = 0;

    // Wave w's partial of head hh for stash slot s of flush buffer buf
    // (8-head kernel: over the wave's K / V rows).
    auto part = [&](int buf, int s, int hh, int w) __attribute__((always_inline)) -> float* {
        if constexpr (OA) return reinterpret_cast<float*>(&sm_k[w][0]) + hh * D;
        else return &sm_o[buf][s][hh][w][0];
    };

    // Matrix-core kernels: the flush runs head-major, thread tid merging
    // head tid / TPH at its EH consecutive dims, so each thread takes the
    // exponentials of one head's wave maxima (not of every head's) and reads
    // its partials as vectors; each (head, dim) gets the same arithmetic.
    constexpr int TPH = MF ? kAttnThreads / G : 1;       // threads per head
    constexpr int EH = MF ? D / TPH : 1;                  // dims per thread
    static_assert(!MF || EH * TPH == D, "head-major flush: whole dims per thread");
    const int fh = MF ? tid / TPH : 0;                    // this thread's head
    const int fd = MF ? (tid % TPH) * EH : 0;             // its first dim

    auto flush = [&]() __attribute__((always_inline)) {
        const int buf = n_flush % NB;
        ++n_flush;
        __syncthreads();
        if constexpr (MF) {
            for (int s = 0; s < n_st; ++s) {
                const int ch = st_first + s;
                float mw[kAttnWaves], lw[kAttnWaves], ow[kAttnWaves][EH];
#pragma unroll
                for (int w = 0; w < kAttnWaves; ++w) {
                    mw[w] = sm_m[buf][s][fh][w];
                    lw[w] = sm_l[buf][s][fh][w];
                    const float* pw = part(buf, s, fh, w) + fd;
#pragma unroll
                    for (int e = 0; e < EH; ++e) ow[w][e] = pw[e];
                }
                float M = mw[0];
#pragma unroll
                for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, mw[w]);
                // no valid key in the chunk: sum and partial stay zero
                const bool any = M != -INFINITY;
                float L = 0.f, O[EH];
#pragma unroll
                for (int e = 0; e < EH; ++e) O[e] = 0.f;
#pragma unroll
                for (int w = 0; w < kAttnWaves; ++w) {
                    const float a = any ? fast_exp2(mw[w] - M) : 0.f;
                    L = fmaf(lw[w], a, L);
#pragma unroll
                    for (int e = 0; e < EH; ++e) O[e] = fmaf(ow[w][e], a, O[e]);
                }
                if (fh >= gv) {
                    // idle head: nothing to keep
                } else if (MODE == kModePartials) {
                    const size_t idx = (size_t)(bh0 + fh) * P.n_chunk + ch;
#pragma unroll
                    for (int e = 0; e < EH; ++e) P.part_o[idx * D + fd + e] = O[e] * vscale;
                    if (fd == 0) {
                        P.part_ml[idx * 2 + 0] = M == -INFINITY ? -INFINITY : M * kLn2;
                        P.part_ml[idx * 2 + 1] = L;
                    }
                } else if (P.wpp == 1) {
                    // the running fold waits in LDS, each (head, dim) with the
                    // threads that merge it (M and L: the head's first one)
                    float fo[EH];
#pragma unroll
                    for (int e = 0; e < EH; ++e) fo[e] = sm_run_o[fh][fd + e];
                    const float fM = sm_run_ml[fh][0], fL = sm_run_ml[fh][1];
#pragma unroll
                    for (int e = 0; e < EH; ++e) {
                        Fold f;
                        f.M = fM;
                        f.L = fL;
                        f.O = fo[e];
                        f.add_sel(M, L, O[e]);
                        sm_run_o[fh][fd + e] = f.O;
                        if (e == 0 && fd == 0) {
                            sm_run_ml[fh][0] = f.M;
                            sm_run_ml[fh][1] = f.L;
                        }
                    }
                } else {
                    const size_t idx = (size_t)(bh0 + fh) * P.n_chunk + ch;
#pragma unroll
                    for (int e = 0; e < EH; ++e) st_agent(P.part_o + idx * D + fd + e, O[e]);
                    if (fd == 0) {
                        st_agent(P.part_ml + idx * 2 + 0, M);
                        st_agent(P.part_ml + idx * 2 + 1, L);
                    }
                }
            }
        } else
        for (int s = 0; s < n_st; ++s) {
            const int ch = st_first + s;
            // every head's wave maxima, sums and partials are read first and
            // merged with selects, not branches (a branch per head would make
            // each head wait for its own LDS reads in turn)
            float Mc[G], Lc[G], Oc[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float mw[kAttnWaves], lw[kAttnWaves], ow[kAttnWaves];
#pragma unroll
                for (int w = 0; w < kAttnWaves; ++w) {
                    mw[w] = sm_m[buf][s][hh][w];
                    lw[w] = sm_l[buf][s][hh][w];
                    ow[w] = t < D ? part(buf, s, hh, w)[t] : 0.f;
                }
                float M = mw[0];
#pragma unroll
                for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, mw[w]);
                // no valid key in the chunk: sum and partial stay zero
                const bool any = M != -INFINITY;
                float L = 0.f, O = 0.f;
#pragma unroll
                for (int w = 0; w < kAttnWaves; ++w) {
                    const float a = any ? fast_exp2(mw[w] - M) : 0.f;
                    L = fmaf(lw[w], a, L);
                    O = fmaf(ow[w], a, O);
                }
                Mc[hh] = M;
                Lc[hh] = L;
                Oc[hh] = O;
            }
            // then each head's chunk partial is kept (idle heads of the 4- and
            // 8-head kernels: nothing to keep)
            if (MODE == kModePartials) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    if (hh >= gv) continue;
                    const size_t idx = (size_t)(bh0 + hh) * P.n_chunk + ch;
                    if (t < D) P.part_o[idx * D + t] = Oc[hh] * vscale;
                    if (tid == 0) {
                        P.part_ml[idx * 2 + 0] = Mc[hh] == -INFINITY ? -INFINITY : Mc[hh] * kLn2;
                        P.part_ml[idx * 2 + 1] = Lc[hh];
                    }
                }
            } else if (P.wpp == 1) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh)
                    if (hh < gv) run[hh].add(Mc[hh], Lc[hh], Oc[hh]);
            } else {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    if (hh >= gv) continue;
                    const size_t idx = (size_t)(bh0 + hh) * P.n_chunk + ch;
                    if (t < D) st_agent(P.part_o + idx * D + t, Oc[hh]);
                    if (tid == 0) {
                        st_agent(P.part_ml + idx * 2 + 0, Mc[hh]);
                        st_agent(P.part_ml + idx * 2 + 1, Lc[hh]);
                    }
                }
            }
        }
        // a single flush buffer: every thread has read it before any wave
        // writes its next chunk's partial (or stages a tile) there
        if constexpr (NB == 1) __syncthreads();
        n_st = 0;
    };

    auto end_chunk = [&](int ch) __attribute__((always_inline)) {
        float l_w[G] = {};
        if constexpr (!MF) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh) l_w[hh] = wave_sum(l_lane[hh]);
        }
        const int buf = n_flush % NB;
        if constexpr (MF) {
            // the running max and sum first (the flushes below read them);
            // head (lane % 16): its max is already the same in its 4 lanes,
            // its sum adds the 4 lanes' shares
            const float lw = xor_sum<32>(xor_sum<16>(l1)) * kPUnscale;
            if (lane < G) {
                sm_m[buf][n_st][lane][wid] = m1;
                sm_l[buf][n_st][lane][wid] = lw;
            }
            m1 = -INFINITY;
            l1 = 0.f;
            if (n_st == 0) st_first = ch;
            // O from the matrix cores (already summed over this wave's
            // keys): every lane writes dim 64 m + l of every head (the
            // 8-head kernel over its own K / V rows: it has read them, and
            // its LDS accesses complete in order)
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
#pragma unroll
                for (int m = 0; m < D / 64; ++m)
                    part(buf, n_st, hh, wid)[64 * m + lane] =
                        pv_acc[hh / 4 * (D / 64) + m][hh % 4] * kPUnscale;
            }
#pragma unroll
            for (int m = 0; m < NACC; ++m) pv_acc[m] = pv4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int hh = 0; hh < (MF ? 0 : G); ++hh) {
            // head by head: sum over the lanes that share this lane's dims,
            // then store, so only one head's exchanges are live at a time
#pragma unroll
            for (int m = LPR; m < kWave; m <<= 1) {
#pragma unroll
                for (int e = 0; e < EPC; ++e) o_acc[hh][e] = xor_sum_rt(o_acc[hh][e], m);
            }
            if (r == 0) {
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    sm_o[buf][n_st][hh][wid][c * EPC + e] = o_acc[hh][e] * kPUnscale;
            }
            if (lane == 0) {
                sm_m[buf][n_st][hh][wid] = m_run[hh];
                sm_l[buf][n_st][hh][wid] = l_w[hh];
            }
            m_run[hh] = -INFINITY;
            l_lane[hh] = 0.f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) o_acc[hh][e] = 0.f;
        }
        if (!MF && n_st == 0) st_first = ch;
        ++n_st;
        if (n_st == kStash) flush();
    };


    // Query heads and new key rotated in-kernel for the fused step (one angle
    // for all); each query scaled by scale*log2(e) and, for an fp8 cache, by
    // the head's K scale (cached keys are scale * code, so the scale moves
    // onto the query once).
    float k_r = k_t;
    float qsc[G];
    {
        double cs = 1.0, sn = 0.0;
        const int half = P.rot >> 1;
        if (rotated) {
            rope_cs(td < half ? td : td - half, P.rot, P.log2_theta, p, cs, sn);
            k_r = rope_rotate(k_t, k_p, td < half, cs, sn);
        }
        const float qmul = P.qscale * kscale;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float q_r = rotated ? rope_rotate(q_t[hh], q_p[hh], td < half, cs, sn) : q_t[hh];
            qsc[hh] = q_r * qmul;
            if constexpr (MF) {              // empty running fold
                if (t < D) sm_run_o[hh][t] = 0.f;
                if (tid == 0) {
                    sm_run_ml[hh][0] = -INFINITY;
                    sm_run_ml[hh][1] = 0.f;
                }
            }
            if (t < D) {
                if constexpr (MF) {          // 16-bit hi + lo parts for the MFMA operand
                    if (t == 0) sm_glogit[hh] = glogit[hh];    // read back in the epilogue
                    constexpr int QT = DT == kF16 ? kF16 : kBF16;
                    const uint16_t hi = round_to_elt<QT>(qsc[hh]);
                    sm_qh[hh][t] = hi;
                    sm_ql[hh][t] = round_to_elt<QT>(qsc[hh] - elt_to_f32<QT>(hi));
                } else {
                    sm_q[hh][t] = qsc[hh];
                }
            }
        }
        if constexpr (MF) {
            if (t < D) {                     // the zero query of idle columns
                sm_qh[G][t] = 0;
                sm_ql[G][t] = 0;
            }
        }
    }

    // The new entry, joined in score space: k_hat, v_hat are the rotated key
    // and the value rounded to the cache element type (fp8: the code of
    // x / scale, the quotient rounded once to float32); its score with every
    // query head is summed now and folded last, after the cached keys.
    S k_hat{}, v_hat{};
    float vh = 0.f;
    if (has_new) {
        float khf = 0.f;
        if (t < D) {
            k_hat = round_to_elt<DT>(DT == kFP8 ? __fdiv_rn(k_r, kscale) : k_r);
            v_hat = round_to_elt<DT>(DT == kFP8 ? __fdiv_rn(v_t, vscale) : v_t);
            khf = elt_to_f32<DT>(k_hat);
            vh = elt_to_f32<DT>(v_hat);
            if constexpr (MF) sm_vh[t] = vh;        // joined head-major in the epilogue
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const float prod = wave_sum(t < D ? qsc[hh] * khf : 0.f);
            if (lane == 0) sm_dot[hh][wid] = prod;
        }
    }
    // Gate logits from the projection (fused step with g_proj): they need
    // only the layer input, so they are summed here, under the first tiles'
    // latency, and used in the epilogue.  Same sum as hswd_gate_proj.
    if (gproj) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float gs = hh < gv ? gate_share(P.gx + (size_t)b * P.hidden,
                                            P.gw + (size_t)(bh0 - b * P.H + hh) * P.hidden,
                                            P.hidden, tid, kAttnThreads)
                               : 0.f;
            gs = wave_sum(gs);
            if (lane == 0) sm_gl[hh][wid] = gs;
        }
    }
    __syncthreads();
    if constexpr (!MF) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
#pragma unroll
            for (int e = 0; e < EPC; ++e) qs[hh][e] = sm_q[hh][c * EPC + e];
        }
    }
    if constexpr (MF) {
        // lanes of heads >= G read the zero row G
        const int hq = lane & 15, kq = lane >> 4;
#pragma unroll
        for (int sl = 0; sl < D / 32; ++sl) {
            qhr[sl] = *reinterpret_cast<const u32x4*>(&sm_qh[hq < G ? hq : G][8 * kq + 32 * sl]);
            qlr[sl] = *reinterpret_cast<const u32x4*>(&sm_ql[hq < G ? hq : G][8 * kq + 32 * sl]);
        }
    }

    // Chunk boundaries fall after every TPW-th item among the full chunks
    // (items are scored in order, each once); every wave has the same items,
    // so the barriers match.
    int left = TPW, ch_cur = c_begin;
    auto after = [&](int j) __attribute__((always_inline)) {
        if (j < n_full_items && --left == 0) {
            end_chunk(ch_cur);
            ++ch_cur;
            left = TPW;
        }
    };
    // Entering each pass, A holds item j and B item j + 1, both requested; a
    // buffer is refilled as soon as it has been scored.  The loop body's
    // loads are unconditional (j + 3 < n_items), so its wait counts keep the
    // other buffer in flight.
    if constexpr (VS1) {
        // one buffer: each tile requests the next one's K and V itself
        for (int j = 0; j < n_items; ++j) {
            compute_tile(kA, vA, j);
            after(j);
        }
    } else {
        int j = 0;
        for (; j + 3 < n_items; j += 2) {
            compute_tile(kA, vA, j);
            after(j);
            load_tile(kA, vA, j + 2);
            compute_tile(kB, vB, j + 1);
            after(j + 1);
            load_tile(kB, vB, j + 3);
        }
        if (j + 2 < n_items) {
            compute_tile(kA, vA, j);
            after(j);
            load_tile(kA, vA, j + 2);
            compute_tile(kB, vB, j + 1);
            after(j + 1);
            compute_tile(kA, vA, j + 2);
            after(j + 2);
        } else if (j + 1 < n_items) {
            compute_tile(kA, vA, j);
            after(j);
            compute_tile(kB, vB, j + 1);
            after(j + 1);
        } else if (j < n_items) {
            compute_tile(kA, vA, j);
            after(j);
        }
    }
    if (c_valid > c_full) end_chunk(c_full);            // the partly valid chunk
    if (n_st > 0) flush();
    // Matrix-core kernels finish head-major too: thread (fh, fd) holds the
    // running fold of head fh at dims fd .. fd + EH - 1 (M and L per head)
    float hM = -INFINITY, hL = 0.f, hO[EH];
#pragma unroll
    for (int e = 0; e < EH; ++e) hO[e] = 0.f;
    if constexpr (MF) {
        if (MODE != kModePartials && P.wpp == 1) {
            // folded in LDS by this thread's own flushes
            hM = sm_run_ml[fh][0];
            hL = sm_run_ml[fh][1];
#pragma unroll
            for (int e = 0; e < EH; ++e) hO[e] = sm_run_o[fh][fd + e];
        }
    }

    if (MODE == kModePartials) {
        // chunks without a valid key are empty partials
        for (int ch = c_valid; ch < c_end; ++ch) {
#pragma unroll
            for (int hh = 0; hh < gv; ++hh) {
                const size_t idx = (size_t)(bh0 + hh) * P.n_chunk + ch;
                if (t < D) P.part_o[idx * D + t] = 0.f;
                if (tid == 0) {
                    P.part_ml[idx * 2 + 0] = -INFINITY;
                    P.part_ml[idx * 2 + 1] = 0.f;
                }
            }
        }
        return;
    }

    if (P.wpp > 1) {
        // Partials cross workgroups (and possibly XCDs).  They are written and
        // read only with agent-scope atomic stores and loads, which go to the
        // device-coherent level themselves, so no L2 write-back or invalidate
        // is needed: each thread waits for its own stores to complete, the
        // barrier makes that true for the whole workgroup, and only then is
        // the arrival counted.  The merging workgroup reads the partials after
        // it has seen the final count.
        wait_stores_complete();
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(&P.counters[pair * npiece + piece], 1,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm_last = prev == (packed ? pack_parts : P.wpp) - 1;
        }
        __syncthreads();
        if (!sm_last) return;

        // Last arrival folds the valid chunks of each head in chunk order, 32
        // partials' loads in flight before any is folded (matrix-core
        // kernels: head-major, 64 partial values in flight per thread).
        if constexpr (MF) {
            if (fh < gv) {
                const float* pml = P.part_ml + (size_t)(bh0 + fh) * P.n_chunk * 2;
                const float* po = P.part_o + (size_t)(bh0 + fh) * P.n_chunk * D + fd;
                constexpr int kB = EH >= 8 ? 8 : 32 / EH;
                int i = 0;
                for (; i + kB <= n_valid_chunks; i += kB) {
                    float xm[kB], xl[kB], xo[kB][EH];
#pragma unroll
                    for (int u = 0; u < kB; ++u) {
                        xm[u] = ld_agent(pml + 2 * (i + u));
                        xl[u] = ld_agent(pml + 2 * (i + u) + 1);
#pragma unroll
                        for (int e = 0; e < EH; ++e) xo[u][e] = ld_agent(po + (size_t)(i + u) * D + e);
                    }
#pragma unroll
                    for (int u = 0; u < kB; ++u) fold_row<EH>(hM, hL, hO, xm[u], xl[u], xo[u]);
                }
                for (; i < n_valid_chunks; ++i) {
                    float xo[EH];
#pragma unroll
                    for (int e = 0; e < EH; ++e) xo[e] = ld_agent(po + (size_t)i * D + e);
                    fold_row<EH>(hM, hL, hO, ld_agent(pml + 2 * i), ld_agent(pml + 2 * i + 1), xo);
                }
            }
        } else
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            if (hh >= gv) continue;
            const float* pml = P.part_ml + (size_t)(bh0 + hh) * P.n_chunk * 2;
            const float* po = P.part_o + (size_t)(bh0 + hh) * P.n_chunk * D + (t < D ? t : 0);
            constexpr int kBatch = 32;
            int i = 0;
            for (; i + kBatch <= n_valid_chunks; i += kBatch) {
                float xm[kBatch], xl[kBatch], xo[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    xm[u] = ld_agent(pml + 2 * (i + u));
                    xl[u] = ld_agent(pml + 2 * (i + u) + 1);
                    xo[u] = ld_agent(po + (size_t)(i + u) * D);
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) run[hh].add(xm[u], xl[u], xo[u]);
            }
            for (; i < n_valid_chunks; ++i)
                run[hh].add(ld_agent(pml + 2 * i), ld_agent(pml + 2 * i + 1),
                            ld_agent(po + (size_t)i * D));
        }
        if (tid == 0)                            // ready for the next call
            __hip_atomic_store(&P.counters[pair * npiece + piece], 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }

    // Join the new entry as a one-key partial (scores summed in the prologue).
    // Matrix-core kernels: head-major, the head's gate computed once.
    if constexpr (MF) {
        const float sn = lds_tree_sum<kAttnWaves>(sm_dot[fh]);
        const float lg = gproj ? lds_tree_sum<kAttnWaves>(sm_gl[fh]) : sm_glogit[fh];
        float vv[EH];
#pragma unroll
        for (int e = 0; e < EH; ++e) vv[e] = sm_vh[fd + e];
        fold_row<EH>(hM, hL, hO, sn, 1.f, vv);
        if (fh < gv) {
            const bool gated = MODE == kModeStep && (gproj || P.gate != nullptr);
            const float gs = gated ? 1.f / (1.f + expf(-lg)) : 1.f;
#pragma unroll
            for (int e = 0; e < EH; ++e) {
                float o = hO[e] / hL;
                if (DT == kFP8) o *= vscale;
                if (gated) o *= gs;
                P.out[(size_t)(bh0 + fh) * D + fd + e] = o;
            }
        }
    } else {
        // every head's LDS reads first
        float s_new[G], logit[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            s_new[hh] = lds_tree_sum<kAttnWaves>(sm_dot[hh]);
            logit[hh] = gproj ? lds_tree_sum<kAttnWaves>(sm_gl[hh]) : glogit[hh];
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            run[hh].add(s_new[hh], 1.f, vh);
            if (t < D && hh < gv) {
                float o = run[hh].O / run[hh].L;
                if (DT == kFP8) o *= vscale;
                if (MODE == kModeStep && (gproj || P.gate != nullptr))
                    o *= 1.f / (1.f + expf(-logit[hh]));
                P.out[(size_t)(bh0 + hh) * D + t] = o;
            }
        }
    }

    if (MODE == kModeStep && npiece > 1) {
        // Several head pieces read this pair's cache: the piece that finishes
        // last writes the entry.  Each piece arrives once (its only or its
        // merging workgroup) after every wave's loads have returned (their
        // values are used before the barrier).
        __syncthreads();
        if (tid == 0) {
            int32_t* ec = P.counters + (size_t)n_pairs * npiece + pair;
            const int prev = __hip_atomic_fetch_add(ec, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            sm_last = prev == npiece - 1;
            if (sm_last) __hip_atomic_store(ec, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!sm_last) return;
    }
    if (MODE == kModeStep) {
        // Every workgroup of this pair has finished reading (one workgroup:
        // the barrier of the last stash flush, which every wave reaches after
        // its last tile; several: the arrival counts), so the ring slot that
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
