// Device helpers shared by the hswd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hswd {

constexpr int kWave = 64;

// Cache element type codes (hswd_dtype).
constexpr int kF32 = 0;
constexpr int kF16 = 1;
constexpr int kBF16 = 2;
constexpr int kFP8 = 3;     // OCP fp8 e4m3 with a per-head scale

template <int DT> struct Storage { using type = uint16_t; };
template <> struct Storage<kF32> { using type = float; };
template <> struct Storage<kFP8> { using type = uint8_t; };

template <int DT> constexpr int elt_bytes() { return DT == kF32 ? 4 : (DT == kFP8 ? 1 : 2); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One lane's chunk of a cache row: 16 bytes, or 8 (fp8 rows in the grouped
// kernels, so a lane holds 8 dims there too).
template <int CB> struct ChunkT;
template <> struct ChunkT<16> { using type = u32x4; };
template <> struct ChunkT<8> { using type = u32x2; };

// K/V tile loads.  A row read by one workgroup only is streamed with the
// non-temporal hint (on MI355X the hinted loads stream from HBM about 10%
// faster than plain ones); rows that several workgroups read close together
// (SHARED) use plain loads, which leave them in L2 for the others.
template <int CB, bool SHARED = false, typename T>
__device__ __forceinline__ typename ChunkT<CB>::type load_kv(const T* p) {
    using C = typename ChunkT<CB>::type;
    if constexpr (SHARED) return *reinterpret_cast<const C*>(p);
    else return __builtin_nontemporal_load(reinterpret_cast<const C*>(p));
}

// ---------------------------------------------------------------------------
// float32 -> cache element, IEEE round to nearest, ties to even, by integer
// arithmetic on the bit pattern.  NaN stays NaN: sign kept, quiet bit set,
// the leading payload bits kept.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    // Adding 0x7fff plus the kept lsb carries into the kept bits exactly when
    // the dropped half is above the midpoint, or at it with an odd lsb; a
    // carry out of the significand bumps the exponent (up to infinity).
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a & 0x7fffffu) >> 13));
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);   // |x| >= 65520: rounds to inf
    if (a >= 0x38800000u) {                                     // |x| >= 2^-14: normal result
        uint32_t r = a - 0x38000000u;                           // exponent bias 127 -> 15
        r += 0x0fffu + ((r >> 13) & 1u);                        // ties to even on 13 dropped bits
        return (uint16_t)(sign | (r >> 13));
    }
    if (a < 0x33000000u) return (uint16_t)sign;                 // |x| < 2^-25: rounds to 0
    // subnormal result: value / 2^-24 = significand >> (126 - exponent)
    uint32_t e = a >> 23;
    uint32_t m = (a & 0x7fffffu) | 0x800000u;
    uint32_t sh = 126u - e;                                     // 14 .. 24
    uint32_t q = m >> sh;
    uint32_t rem = m & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1u);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return (uint16_t)(sign | q);
}

// float32 -> OCP fp8 e4m3 (bias 7, 3 fraction bits, no infinities, largest
// finite 448), round to nearest, ties to even, saturating: |x| >= 448 and
// infinities become +-448.  NaN stays NaN (code 0x7f with the sign).
__device__ __forceinline__ uint8_t f32_to_fp8_rne_sat(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint8_t)(sign | 0x7fu);
    if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);      // |x| >= 448
    if (a >= 0x3c800000u) {                                     // |x| >= 2^-6: normal
        uint32_t r = a - 0x3c000000u;                           // exponent bias 127 -> 7
        r += 0x7ffffu + ((r >> 20) & 1u);                       // ties to even on 20 bits
        uint32_t code = r >> 20;
        return (uint8_t)(sign | (code > 0x7eu ? 0x7eu : code));
    }
    if (a < 0x39800000u) return (uint8_t)sign;                  // |x| < 2^-12: rounds to 0
    // subnormal result: value / 2^-9 = significand >> (141 - exponent)
    uint32_t e = a >> 23;
    uint32_t m = (a & 0x7fffffu) | 0x800000u;
    uint32_t sh = 141u - e;                                     // 21 .. 26
    uint32_t q = m >> sh;
    uint32_t rem = m & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1u);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return (uint8_t)(sign | q);
}

// Two fp8 e4m3 codes (bytes 0-1 or 2-3 of w) to float32, by the hardware
// conversion (gfx950 decodes the OCP format; checked on all 256 codes).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 fp8x2_to_f32(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    _Float16 f = __builtin_bit_cast(_Float16, h);
    return (float)f;
}

template <int DT>
__device__ __forceinline__ typename Storage<DT>::type round_to_elt(float x) {
    if constexpr (DT == kF32) return x;
    else if constexpr (DT == kF16) return f32_to_f16_rne(x);
    else if constexpr (DT == kFP8) return f32_to_fp8_rne_sat(x);
    else return f32_to_bf16_rne(x);
}

template <int DT>
__device__ __forceinline__ float elt_to_f32(typename Storage<DT>::type s) {
    if constexpr (DT == kF32) return s;
    else if constexpr (DT == kF16) return f16_bits_to_f32(s);
    else if constexpr (DT == kFP8) return fp8x2_to_f32((uint32_t)s, false).x;
    else return bf16_bits_to_f32(s);
}

// Unpack one 16-byte chunk of cache elements into floats (EPC of them).
template <int DT>
__device__ __forceinline__ void unpack_chunk(const u32x4& w, float* f) {
    if constexpr (DT == kFP8) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f32x2 lo = fp8x2_to_f32(u[j], false), hi = fp8x2_to_f32(u[j], true);
            f[4 * j] = lo.x; f[4 * j + 1] = lo.y; f[4 * j + 2] = hi.x; f[4 * j + 3] = hi.y;
        }
    } else if constexpr (DT == kF32) {
        f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
        f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
    } else if constexpr (DT == kBF16) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(u[j] << 16);
            f[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
        }
    } else {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = f16_bits_to_f32((uint16_t)(u[j] & 0xffffu));
            f[2 * j + 1] = f16_bits_to_f32((uint16_t)(u[j] >> 16));
        }
    }
}

// Two fp8 e4m3 codes (bytes 0-1 or 2-3 of w) to two bf16 values packed in a
// word (the first code in the low half), by the gfx950 scaled conversion
// with scale 1: exact, as every e4m3 value is a bf16 value.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

// Eight fp8 codes (byte order) -> eight bf16 values, exactly, two per
// conversion.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(const u32x2& w) {
    return u32x4{fp8x2_to_bf16x2(w.x, false), fp8x2_to_bf16x2(w.x, true),
                 fp8x2_to_bf16x2(w.y, false), fp8x2_to_bf16x2(w.y, true)};
}

// Two fp8 e4m3 codes (bytes 0-1 or 2-3 of w) to two fp16 values packed in a
// word (the first code in the low half), by the gfx950 scaled conversion
// with scale 1: exact, as every e4m3 value is an fp16 value.
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w, bool hi) {
    return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
              : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}

// Eight fp8 codes (a lane's chunk of a grouped kernel's row) as eight fp16
// values, in element order; exact, since every e4m3 value is an fp16 value.
__device__ __forceinline__ u32x4 fp8x8_to_f16x8(const u32x2& w) {
    return u32x4{fp8x2_to_f16x2(w.x, false), fp8x2_to_f16x2(w.x, true),
                 fp8x2_to_f16x2(w.y, false), fp8x2_to_f16x2(w.y, true)};
}

// Unpack one 8-byte chunk of fp8 codes into 8 floats, in byte order.
template <int DT>
__device__ __forceinline__ void unpack_chunk(const u32x2& w, float* f) {
    static_assert(DT == kFP8, "8-byte chunks hold fp8 codes");
    const uint32_t u[2] = {w.x, w.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const f32x2 lo = fp8x2_to_f32(u[j], false), hi = fp8x2_to_f32(u[j], true);
        f[4 * j] = lo.x; f[4 * j + 1] = lo.y; f[4 * j + 2] = hi.x; f[4 * j + 3] = hi.y;
    }
}

// ---------------------------------------------------------------------------
// Wave exchanges between lane l and lane l ^ M, all in the VALU:
//   M = 1, 2:   DPP quad permutations;
//   M = 4:      DPP row shifts by 4 (left for lanes with bit 2 clear, right
//               for the others) and a select;
//   M = 8:      DPP row rotation by 8 (rows of 16 lanes);
//   M = 16, 32: the gfx950 permlane swaps.  v_permlane{16,32}_swap(a, b)
//               leaves, in a lane with bit M clear, (a[l], a[l + M]) and in
//               a lane with it set, (b[l - M], b[l]).  With a = b = v the two
//               results are the values of both lanes of the pair, so their
//               sum or max is the pair's (addition and max are commutative:
//               the same bits as v + v[l ^ M]) without a select.
// xor_sum / xor_max return v op v[l ^ M]; xor_lane the partner's value.
// ---------------------------------------------------------------------------
namespace dpp {
constexpr int kQuad10 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuad23 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowShl4 = 0x104;   // lane l reads lane l + 4 of its row
constexpr int kRowShr4 = 0x114;   // lane l reads lane l - 4 of its row
constexpr int kRowRor8 = 0x128;   // lane l reads lane l ^ 8 of its row
template <int CTRL>
__device__ __forceinline__ float mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
}  // namespace dpp

// The two results of a permlane swap of (a, b) over distance M (16 or 32).
template <int M>
__device__ __forceinline__ void lane_swap(float a, float b, float& r0, float& r1) {
    static_assert(M == 16 || M == 32, "swap distance");
    if constexpr (M == 16) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    } else {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
        r0 = __uint_as_float(r[0]);
        r1 = __uint_as_float(r[1]);
    }
}

template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "mask");
    if constexpr (M == 1) {
        return dpp::mov<dpp::kQuad10>(v);
    } else if constexpr (M == 2) {
        return dpp::mov<dpp::kQuad23>(v);
    } else if constexpr (M == 4) {
        const float up = dpp::mov<dpp::kRowShr4>(v), dn = dpp::mov<dpp::kRowShl4>(v);
        return (__lane_id() & 4) ? up : dn;
    } else if constexpr (M == 8) {
        return dpp::mov<dpp::kRowRor8>(v);
    } else {
        float r0, r1;
        lane_swap<M>(v, v, r0, r1);
        return (__lane_id() & M) ? r0 : r1;
    }
}

template <int M>
__device__ __forceinline__ float xor_sum(float v) {
    if constexpr (M == 16 || M == 32) {
        float r0, r1;
        lane_swap<M>(v, v, r0, r1);
        return r0 + r1;
    } else {
        return v + xor_lane<M>(v);
    }
}

template <int M>
__device__ __forceinline__ float xor_max(float v) {
    if constexpr (M == 16 || M == 32) {
        float r0, r1;
        lane_swap<M>(v, v, r0, r1);
        return fmaxf(r0, r1);
    } else {
        return fmaxf(v, xor_lane<M>(v));
    }
}

// Mask known at compile time after unrolling (the loops that call these run
// over powers of two with constant bounds).
__device__ __forceinline__ float xor_sum_rt(float v, int m) {
    switch (m) {
        case 1: return xor_sum<1>(v);
        case 2: return xor_sum<2>(v);
        case 4: return xor_sum<4>(v);
        case 8: return xor_sum<8>(v);
        case 16: return xor_sum<16>(v);
        default: return xor_sum<32>(v);
    }
}

__device__ __forceinline__ float xor_max_rt(float v, int m) {
    switch (m) {
        case 1: return xor_max<1>(v);
        case 2: return xor_max<2>(v);
        case 4: return xor_max<4>(v);
        case 8: return xor_max<8>(v);
        case 16: return xor_max<16>(v);
        default: return xor_max<32>(v);
    }
}

// Value of lane `src` (any lane): ds_bpermute.
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

__device__ __forceinline__ float wave_sum(float v) {
    v = xor_sum<32>(v); v = xor_sum<16>(v); v = xor_sum<8>(v);
    v = xor_sum<4>(v); v = xor_sum<2>(v); v = xor_sum<1>(v);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    v = xor_max<32>(v); v = xor_max<16>(v); v = xor_max<8>(v);
    v = xor_max<4>(v); v = xor_max<2>(v); v = xor_max<1>(v);
    return v;
}

// Agent-scope (whole GPU) relaxed atomic store / load of a float.
__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every vector memory operation this thread issued, stores
// included, has completed.  The asm's memory clobber also keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void wait_stores_complete() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pairwise-tree sum of N values in LDS (fixed order: deterministic).
template <int N>
__device__ __forceinline__ float lds_tree_sum(const float* a) {
    if constexpr (N == 1) return a[0];
    else return lds_tree_sum<N / 2>(a) + lds_tree_sum<N / 2>(a + N / 2);
}

// This thread's share of one gate logit, x . w_g[h, :]: the terms i = tid,
// tid + nthreads, ... in order.  The head-gate projection of the pages' model
// maps the layer's post-norm input (hidden 2048) to one logit per head.
// Loads go out 16 at a time before any is used, so the share costs about one
// memory latency.  Callers sum the shares of 256 threads by wave_sum and a
// 4-wave tree, so the standalone projection and the fused layer step give the
// same bits.
__device__ __forceinline__ float gate_share(const float* x, const float* w_row, int hidden,
                                            int tid, int nthreads) {
    constexpr int kBatch = 8;
    float acc = 0.f;
    for (int i0 = tid; i0 < hidden; i0 += kBatch * nthreads) {
        float xv[kBatch], wv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = i0 + u * nthreads;
            xv[u] = i < hidden ? x[i] : 0.f;
            wv[u] = i < hidden ? w_row[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (i0 + u * nthreads < hidden) acc = fmaf(xv[u], wv[u], acc);
    }
    return acc;
}

// ---------------------------------------------------------------------------
// RoPE of element t of one head vector x[0..D) at position p: the pair
// (x[i], x[i + rot/2]) turns by p * theta^(-2i/rot); dims >= rot pass.  The
// inverse frequency is 2^(-(2i/rot) * log2(theta)); angle, sine, cosine and
// rotation are in double precision, rounded once to float.  The rotation's
// fused multiply-adds are written out, so every caller gets the same bits.
// ---------------------------------------------------------------------------
// Cosine and sine of pair i's angle at position p.
__device__ __forceinline__ void rope_cs(int i, int rot, double log2_theta, int p, double& c,
                                        double& s) {
    const double inv = exp2(-(2.0 * (double)i / (double)rot) * log2_theta);
    const double a = (double)p * inv;
    sincos(a, &s, &c);
}

// Element t of the rotated pair from x[t] and its partner x[t +- rot/2]
// (lower: t < rot/2, so x[t] is the pair's first component).
__device__ __forceinline__ float rope_rotate(float xt, float xpart, bool lower, double c,
                                            double s) {
    const double x0 = lower ? (double)xt : (double)xpart;
    const double x1 = lower ? (double)xpart : (double)xt;
    const double r = lower ? __fma_rn(x0, c, -(x1 * s)) : __fma_rn(x1, c, x0 * s);
    return (float)r;
}

// Partner dim of t under RoPE over the first `rot` dims (t itself past rot).
__device__ __forceinline__ int rope_partner(int t, int rot) {
    const int half = rot >> 1;
    return t >= rot ? t : (t < half ? t + half : t - half);
}

__device__ __forceinline__ float rope_elem(const float* x, int t, int rot, double log2_theta,
                                           int p) {
    if (t >= rot) return x[t];
    const int half = rot >> 1;
    double c, s;
    rope_cs(t < half ? t : t - half, rot, log2_theta, p, c, s);
    return rope_rotate(x[t], x[rope_partner(t, rot)], t < half, c, s);
}

}  // namespace hswd
