/*
 * hswd_oracle.c -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * A plain, slow, fp64 CPU statement of one decode step of hybrid
 * sliding-window / full attention.  Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load this library; the GPU path never
 * links, calls or reads it, and it shares no code with the GPU path.
 *
 * Sources (web pages; each citation names the page and the part of it):
 *   [vLLM-Omni/join]   vLLM-Omni fork commit log (tea.kyle-merritt.com,
 *                      anodyine/vllm-omni), the commit that joins the new
 *                      token in score space and keeps a 511-slot ring.
 *   [vLLM-Omni/export] same log, the commit exporting one decode step with
 *                      per-layer-type KV caches and moving the head gate.
 *   [vLLM-Omni/model]  same log, the commit adding the Spark-X2.5 model and
 *                      listing its three traits (hybrid layers, per-type
 *                      RoPE, head-wise sigmoid gate).
 *   [TensorFold#608]   TensorFold pull request 608 "Qwen3.8-27B on CUDA",
 *                      review thread on split decode attention and its merge.
 *
 * Readings taken where the pages are silent:
 *   - softmax scale is a parameter (1/sqrt(head_dim) by default);
 *   - RoPE pairs element i with i + rot/2 ("rotate half") unless
 *     `interleaved` asks for pairs (2i, 2i+1); inverse frequencies run over
 *     the rotary width: inv_i = theta^(-2i/rot);
 *   - pos is the 0-based position of the new token = number of earlier
 *     tokens; a ring of n_slots holds the last min(pos, n_slots) keys, and
 *     slots s < min(pos, n_slots) are the valid ones;
 *   - the new key is rotated, rounded to fp32, then rounded to the cache
 *     element type (round to nearest, ties to even) before it is scored, so
 *     the score-space join sees exactly the entry that is stored;
 *   - the gate multiplies each head's attention output by 1/(1+exp(-g)).
 *
 * Everything is computed in double precision from the exact values the
 * cache element type holds.  No blocking, fusion or reordering beyond the
 * definitions.  Parallelism: OpenMP over (stream, query head) only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_FP8 = 3 };

static int elt_bytes(int dtype) { return dtype == ORC_F32 ? 4 : (dtype == ORC_FP8 ? 1 : 2); }

/* ------------------------------------------------------------------------ */
/* Rounding float32 -> binary16 / bfloat16, round to nearest, ties to even. */
/* Written from the definition: the result is the representable number     */
/* nearest to x on the target format's grid, ties going to the even         */
/* significand; values at or past the midpoint between the largest finite  */
/* number and the next power of two become infinity.  NaN stays NaN (sign   */
/* kept, quiet bit set, leading payload bits kept).                          */
/* ------------------------------------------------------------------------ */

/* Round |x| (finite, non-negative) to a grid with `mant_bits` fraction bits
 * and minimum normal exponent `emin`; returns the rounded magnitude.  The
 * spacing of representable numbers at |x| is 2^(max(e, emin) - mant_bits)
 * where 2^e <= |x| < 2^(e+1).  rint() rounds to nearest, ties to even, in the
 * default floating-point environment. */
static double round_to_grid(double ax, int mant_bits, int emin)
{
    if (ax == 0.0) return 0.0;
    int e;
    frexp(ax, &e);           /* ax = f * 2^e with 0.5 <= f < 1, so 2^(e-1) <= ax */
    int exp2 = e - 1;
    if (exp2 < emin) exp2 = emin;
    double quantum = ldexp(1.0, exp2 - mant_bits);
    return rint(ax / quantum) * quantum;   /* the division by a power of two is exact */
}

uint16_t orc_f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u | ((u & 0x7fffffu) >> 13));
    double ax = fabs((double)x);
    /* largest finite binary16 is 65504 = (2 - 2^-10) * 2^15; the midpoint to
     * 2^16 is 65520, and ties go to the even significand, i.e. to 2^16 = inf. */
    if (ax >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    double r = round_to_grid(ax, 10, -14);
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14))                       /* subnormal: r = m * 2^-24 */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    int e;
    double f = frexp(r, &e);                       /* r = f * 2^e, 0.5 <= f < 1 */
    uint16_t biased = (uint16_t)(e - 1 + 15);
    uint16_t mant = (uint16_t)((f * 2.0 - 1.0) * 1024.0);
    return (uint16_t)(sign | (biased << 10) | mant);
}

uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
    double ax = fabs((double)x);
    /* largest finite bfloat16 is (2 - 2^-7) * 2^127; the midpoint to 2^128 is
     * (2 - 2^-8) * 2^127, which rounds to the even significand, i.e. to inf. */
    if (ax >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7f80u);
    double r = round_to_grid(ax, 7, -126);
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -126))                      /* subnormal: r = m * 2^-133 */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -133)));
    int e;
    double f = frexp(r, &e);
    uint16_t biased = (uint16_t)(e - 1 + 127);
    uint16_t mant = (uint16_t)((f * 2.0 - 1.0) * 128.0);
    return (uint16_t)(sign | (biased << 7) | mant);
}

/* float32 -> OCP fp8 e4m3 (4 exponent bits, bias 7, 3 fraction bits; no
 * infinities; S.1111.111 is NaN; largest finite 448), round to nearest, ties
 * to even, saturating: finite values and infinities that would round past
 * 448 become +-448.  NaN stays NaN (0x7f with the sign). */
uint8_t orc_f32_to_fp8(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if (isnan(x)) return (uint8_t)(sign | 0x7fu);
    double ax = fabs((double)x);
    double r = isinf(x) ? 448.0 : round_to_grid(ax, 3, -6);
    if (r > 448.0) r = 448.0;
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6))                        /* subnormal: r = m * 2^-9 */
        return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    int e;
    double f = frexp(r, &e);
    uint8_t biased = (uint8_t)(e - 1 + 7);
    uint8_t mant = (uint8_t)((f * 2.0 - 1.0) * 8.0);
    return (uint8_t)(sign | (biased << 3) | mant);
}

/* Exact value of an OCP fp8 e4m3 code. */
double orc_fp8_value(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 0xf, m = c & 0x7;
    double v;
    if (e == 0xf && m == 0x7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* Exact value of a binary16 bit pattern. */
double orc_f16_value(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0x1f) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -24);
    else v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

/* Exact value of a bfloat16 bit pattern (the upper half of a float32). */
double orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Element `idx` of an array of cache element type `dtype`, as a double. */
static double load_elt(const void* base, int dtype, size_t idx)
{
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    if (dtype == ORC_FP8) return orc_fp8_value(((const uint8_t*)base)[idx]);
    uint16_t h = ((const uint16_t*)base)[idx];
    return dtype == ORC_F16 ? orc_f16_value(h) : orc_bf16_value(h);
}

/* Round a float32 to the cache element type and store it at `idx`
 * (fp8: with saturation). */
static void store_elt(void* base, int dtype, size_t idx, float x)
{
    if (dtype == ORC_F32) ((float*)base)[idx] = x;
    else if (dtype == ORC_FP8) ((uint8_t*)base)[idx] = orc_f32_to_fp8(x);
    else if (dtype == ORC_F16) ((uint16_t*)base)[idx] = orc_f32_to_f16(x);
    else ((uint16_t*)base)[idx] = orc_f32_to_bf16(x);
}

/* Bulk conversions for the tests. */
void orc_round_f32_to(int dtype, const float* x, size_t n, void* out)
{
    #pragma omp parallel for schedule(static) if (n > 65536)
    for (size_t i = 0; i < n; ++i) store_elt(out, dtype, i, x[i]);
}

void orc_decode(int dtype, const void* x, size_t n, double* out)
{
    #pragma omp parallel for schedule(static) if (n > 65536)
    for (size_t i = 0; i < n; ++i) out[i] = load_elt(x, dtype, i);
}

/* ------------------------------------------------------------------------ */
/* Slot and mask  [vLLM-Omni/join]: position t of a ring of n_slots lives   */
/* in slot t mod n_slots; a ring is never reordered; slots not yet written  */
/* are masked.  An append cache writes position t at row t.                  */
/* ------------------------------------------------------------------------ */
void orc_slot_mask(int B, int n_slots, int ring, const int32_t* pos,
                   int32_t* slot, uint8_t* mask /* [B][n_slots] */)
{
    for (int b = 0; b < B; ++b) {
        int p = pos[b];
        slot[b] = ring ? p % n_slots : p;
        int n_valid = p < n_slots ? p : n_slots;
        for (int s = 0; s < n_slots; ++s) mask[(size_t)b * n_slots + s] = (uint8_t)(s < n_valid);
    }
}

/* ------------------------------------------------------------------------ */
/* RoPE  [vLLM-Omni/model]: sliding layers rotate all head dims at theta    */
/* 1e4, full layers the first quarter at theta 5e6.  Angle a_i = pos*inv_i, */
/* inv_i = theta^(-2i/rot), rotation of the pair (x_i, x_{i+rot/2}) by a_i; */
/* dims at or past rot are left as they are.                                */
/* ------------------------------------------------------------------------ */
void orc_rope(double* out, const float* x, int D, int rot, double theta,
              int64_t pos, int interleaved)
{
    for (int j = 0; j < D; ++j) out[j] = (double)x[j];
    int half = rot / 2;
    for (int i = 0; i < half; ++i) {
        double inv = pow(theta, -2.0 * (double)i / (double)rot);
        double a = (double)pos * inv;
        double c = cos(a), s = sin(a);
        int i0 = interleaved ? 2 * i : i;
        int i1 = interleaved ? 2 * i + 1 : i + half;
        double x0 = (double)x[i0], x1 = (double)x[i1];
        out[i0] = x0 * c - x1 * s;
        out[i1] = x1 * c + x0 * s;
    }
}

/* Apply orc_rope to n vectors of D floats; vector v uses pos[v / per_pos]. */
void orc_rope_batch(double* out, const float* x, int n, int per_pos, int D,
                    int rot, double theta, const int32_t* pos, int interleaved)
{
    for (int v = 0; v < n; ++v)
        orc_rope(out + (size_t)v * D, x + (size_t)v * D, D, rot, theta,
                 (int64_t)pos[v / per_pos], interleaved);
}

/* ------------------------------------------------------------------------ */
/* Attention of one query over a key set  [vLLM-Omni/join]: the cached keys */
/* (rows 0..n-1 of one (stream, kv head) block) and the new entry.  Scores  */
/* s_j = scale * q.K_j, s_new = scale * q.k_new; weights exp(s - max);      */
/* output = sum(w V) / sum(w).  Scoring the new entry on its own and        */
/* joining the two score vectors is the same set of numbers as appending    */
/* the key to the cache; the definition below is that plain set.            */
/* ------------------------------------------------------------------------ */
void orc_attend(double* o, const double* q, const void* kc, const void* vc,
                int dtype, int n, int D, const double* k_new,
                const double* v_new, double scale, double ks, double vs)
{
    double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double s_new = 0.0;
    for (int d = 0; d < D; ++d) s_new += q[d] * k_new[d];
    s_new *= scale;
    double m = s_new;
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += q[d] * (ks * load_elt(kc, dtype, (size_t)j * D + d));
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    double w_new = exp(s_new - m);
    double l = w_new;
    for (int d = 0; d < D; ++d) o[d] = w_new * v_new[d];
    for (int j = 0; j < n; ++j) {
        double w = exp(s[j] - m);
        l += w;
        for (int d = 0; d < D; ++d) o[d] += w * (vs * load_elt(vc, dtype, (size_t)j * D + d));
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
    free(s);
}

/* ------------------------------------------------------------------------ */
/* Split-K form  [TensorFold#608]: the key range is cut into contiguous     */
/* chunks; each chunk gives a partial (m_c, l_c, o_c) with                  */
/* m_c = max s, l_c = sum exp(s - m_c), o_c = sum exp(s - m_c) V (not yet   */
/* divided); the partials are merged by rescaling to the common maximum.    */
/* An empty chunk is (m = -inf, l = 0, o = 0) and contributes nothing.      */
/* ------------------------------------------------------------------------ */
void orc_partial(double* m_out, double* l_out, double* o_out, const double* q,
                 const void* kc, const void* vc, int dtype, int j0, int j1,
                 int D, double scale, double ks, double vs)
{
    for (int d = 0; d < D; ++d) o_out[d] = 0.0;
    if (j1 <= j0) { *m_out = -INFINITY; *l_out = 0.0; return; }
    int n = j1 - j0;
    double* s = (double*)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int j = j0; j < j1; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += q[d] * (ks * load_elt(kc, dtype, (size_t)j * D + d));
        s[j - j0] = scale * acc;
        if (s[j - j0] > m) m = s[j - j0];
    }
    double l = 0.0;
    for (int j = j0; j < j1; ++j) {
        double w = exp(s[j - j0] - m);
        l += w;
        for (int d = 0; d < D; ++d) o_out[d] += w * (vs * load_elt(vc, dtype, (size_t)j * D + d));
    }
    *m_out = m;
    *l_out = l;
    free(s);
}

/* Merge n partials: M = max m_i over non-empty partials,
 * L = sum l_i exp(m_i - M), out = sum o_i exp(m_i - M) / L. */
void orc_merge(double* out, const double* m, const double* l, const double* o,
               int n, int D)
{
    double M = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (l[i] > 0.0 && m[i] > M) M = m[i];
    double L = 0.0;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (int i = 0; i < n; ++i) {
        if (!(l[i] > 0.0)) continue;               /* empty partial */
        double w = exp(m[i] - M);
        L += l[i] * w;
        for (int d = 0; d < D; ++d) out[d] += o[(size_t)i * D + d] * w;
    }
    for (int d = 0; d < D; ++d) out[d] /= L;
}

/* Same key set as orc_attend, computed as chunks [bounds[c], bounds[c+1])
 * of the cached rows plus the new entry as a one-key partial, then merged. */
void orc_attend_split(double* o, const double* q, const void* kc, const void* vc,
                      int dtype, const int32_t* bounds, int n_chunks, int D,
                      const double* k_new, const double* v_new, double scale, double ks,
                      double vs)
{
    int n = n_chunks + 1;
    double* m = (double*)malloc(sizeof(double) * (size_t)n);
    double* l = (double*)malloc(sizeof(double) * (size_t)n);
    double* po = (double*)malloc(sizeof(double) * (size_t)n * D);
    for (int c = 0; c < n_chunks; ++c)
        orc_partial(&m[c], &l[c], po + (size_t)c * D, q, kc, vc, dtype,
                    bounds[c], bounds[c + 1], D, scale, ks, vs);
    double s_new = 0.0;
    for (int d = 0; d < D; ++d) s_new += q[d] * k_new[d];
    m[n_chunks] = scale * s_new;
    l[n_chunks] = 1.0;                              /* exp(s_new - s_new) */
    for (int d = 0; d < D; ++d) po[(size_t)n_chunks * D + d] = v_new[d];
    orc_merge(o, m, l, po, n, D);
    free(m); free(l); free(po);
}

/* ------------------------------------------------------------------------ */
/* Head gate  [vLLM-Omni/model], [vLLM-Omni/export]: each head's attention  */
/* output is scaled by the sigmoid of its gate logit.                       */
/* ------------------------------------------------------------------------ */
double orc_sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

void orc_head_gate(double* out, const double* o, const float* g, int B, int H, int D)
{
    for (int bh = 0; bh < B * H; ++bh) {
        double s = orc_sigmoid((double)g[bh]);
        for (int d = 0; d < D; ++d) out[(size_t)bh * D + d] = o[(size_t)bh * D + d] * s;
    }
}

/* Gate projection  [vLLM-Omni/model], [vLLM-Omni/export]: g_proj maps the  */
/* layer's post-norm input (hidden 2048) to one logit per head; the weight   */
/* is stored a row per head, [H, hidden]: logits[b][h] = sum_i x[b][i]*w[h][i].*/
void orc_gate_proj(double* logits, const float* x, const float* w, int B, int hidden, int H)
{
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int i = 0; i < hidden; ++i)
                acc += (double)x[(size_t)b * hidden + i] * (double)w[(size_t)h * hidden + i];
            logits[(size_t)b * H + h] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Write the new entry  [vLLM-Omni/join]: each layer returns only the new   */
/* K/V entry, which goes into its ring slot (pos mod n_slots) or append row */
/* (pos).  Returns -4 if an append position is at or past the capacity, and */
/* skips that stream's write.                                               */
/* ------------------------------------------------------------------------ */
int orc_write_entry(int B, int Hkv, int D, int n_slots, int dtype, int ring,
                    const int32_t* pos, const void* k_hat, const void* v_hat,
                    void* k_cache, void* v_cache)
{
    int eb = elt_bytes(dtype), status = 0;
    for (int b = 0; b < B; ++b) {
        int p = pos[b];
        if (!ring && p >= n_slots) { status = -4; continue; }
        int row = ring ? p % n_slots : p;
        for (int g = 0; g < Hkv; ++g) {
            size_t dst = (((size_t)b * Hkv + g) * n_slots + row) * D;
            size_t src = ((size_t)b * Hkv + g) * D;
            memcpy((char*)k_cache + dst * eb, (const char*)k_hat + src * eb, (size_t)eb * D);
            memcpy((char*)v_cache + dst * eb, (const char*)v_hat + src * eb, (size_t)eb * D);
        }
    }
    return status;
}

/* ------------------------------------------------------------------------ */
/* One layer step for a batch of streams.                                   */
/*                                                                          */
/*   q [B,H,D], k [B,Hkv,D], v [B,Hkv,D] : float32 projections of the new   */
/*     token (k, q not yet rotated);                                         */
/*   gate [B,H] float32 logits, or NULL for no gate;                         */
/*   k_cache, v_cache [B,Hkv,n_slots,D] of `dtype`: ring (ring != 0) or      */
/*     append cache; updated in place with the new entry when write != 0;   */
/*   pos [B] int32.                                                          */
/* Outputs (any may be NULL):                                                */
/*   out [B,H,D] gated output, o_pre [B,H,D] output before the gate,         */
/*   q_rot [B,H,D], k_rot32 [B,Hkv,D] (the rotated key rounded to float32),  */
/*   k_hat, v_hat [B,Hkv,D] of `dtype` (the entry that is written).          */
/* Returns 0, or -4 when an append position is at or past the capacity      */
/* (that stream's write is skipped, as the GPU path does).                   */
/* Steps, in order: rotate q and k; round the new entry; attend over the    */
/* valid cached keys plus the new entry; gate; then write the entry (the    */
/* write follows the read because a ring's slot pos mod n_slots still holds */
/* position pos - n_slots, which is inside the current window).             */
/* ------------------------------------------------------------------------ */
int orc_layer_step(int B, int H, int Hkv, int D, int n_slots, int dtype, int ring,
                   int rot, double theta, double scale, int interleaved,
                   const int32_t* pos, const float* q, const float* k, const float* v,
                   const float* gate, void* k_cache, void* v_cache, int write,
                   const float* kv_scale,
                   double* out, double* o_pre, double* q_rot, float* k_rot32,
                   void* k_hat, void* v_hat)
{
    int G = H / Hkv;
    int eb = elt_bytes(dtype);
    size_t nkv = (size_t)B * Hkv * D;
    double* qr = (double*)malloc(sizeof(double) * (size_t)B * H * D);
    double* kr = (double*)malloc(sizeof(double) * nkv);
    float* kr32 = (float*)malloc(sizeof(float) * nkv);
    void* kh = malloc((size_t)eb * nkv);
    void* vh = malloc((size_t)eb * nkv);
    double* khd = (double*)malloc(sizeof(double) * nkv);
    double* vhd = (double*)malloc(sizeof(double) * nkv);
    double* opre = (double*)malloc(sizeof(double) * (size_t)B * H * D);

    orc_rope_batch(qr, q, B * H, H, D, rot, theta, pos, interleaved);
    orc_rope_batch(kr, k, B * Hkv, Hkv, D, rot, theta, pos, interleaved);
    for (size_t i = 0; i < nkv; ++i) kr32[i] = (float)kr[i];
    /* With per-head scales (kv_scale [2][Hkv]: K then V; NULL = 1), a cached
     * value is scale * decode(code) and the entry stored is the code of
     * x / scale, the quotient rounded once to float32. */
    float* kq = (float*)malloc(sizeof(float) * nkv);
    float* vq = (float*)malloc(sizeof(float) * nkv);
    for (size_t i = 0; i < nkv; ++i) {
        int g = (int)((i / (size_t)D) % (size_t)Hkv);
        double ks = kv_scale ? (double)kv_scale[g] : 1.0;
        double vs = kv_scale ? (double)kv_scale[Hkv + g] : 1.0;
        kq[i] = (float)((double)kr32[i] / ks);
        vq[i] = (float)((double)v[i] / vs);
    }
    orc_round_f32_to(dtype, kq, nkv, kh);
    orc_round_f32_to(dtype, vq, nkv, vh);
    orc_decode(dtype, kh, nkv, khd);
    orc_decode(dtype, vh, nkv, vhd);
    for (size_t i = 0; i < nkv; ++i) {
        int g = (int)((i / (size_t)D) % (size_t)Hkv);
        if (kv_scale) {
            khd[i] *= (double)kv_scale[g];
            vhd[i] *= (double)kv_scale[Hkv + g];
        }
    }
    free(kq); free(vq);

    int status = 0;
    /* attend: every (stream, query head) reads the cache before any write */
    #pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        int b = bh / H, h = bh % H, g = h / G;
        int p = pos[b];
        /* ring: the last min(p, n_slots) positions; append: rows 0..p-1
         * (bounded by the capacity, which the write check reports) */
        int n = p < n_slots ? p : n_slots;
        size_t blk = ((size_t)b * Hkv + g) * (size_t)n_slots * D;
        orc_attend(opre + (size_t)bh * D, qr + (size_t)bh * D,
                   (const char*)k_cache + blk * eb, (const char*)v_cache + blk * eb,
                   dtype, n, D, khd + ((size_t)b * Hkv + g) * D,
                   vhd + ((size_t)b * Hkv + g) * D, scale,
                   kv_scale ? (double)kv_scale[g] : 1.0,
                   kv_scale ? (double)kv_scale[Hkv + g] : 1.0);
    }

    if (o_pre) memcpy(o_pre, opre, sizeof(double) * (size_t)B * H * D);
    if (out) {
        if (gate) orc_head_gate(out, opre, gate, B, H, D);
        else memcpy(out, opre, sizeof(double) * (size_t)B * H * D);
    }
    if (q_rot) memcpy(q_rot, qr, sizeof(double) * (size_t)B * H * D);
    if (k_rot32) memcpy(k_rot32, kr32, sizeof(float) * nkv);
    if (k_hat) memcpy(k_hat, kh, (size_t)eb * nkv);
    if (v_hat) memcpy(v_hat, vh, (size_t)eb * nkv);

    if (write) status = orc_write_entry(B, Hkv, D, n_slots, dtype, ring, pos, kh, vh, k_cache, v_cache);

    free(qr); free(kr); free(kr32); free(kh); free(vh); free(khd); free(vhd); free(opre);
    return status;
}

/* One (stream, query head) of a layer step, for sampled checks of large
 * workloads: q_rot (D doubles), the (stream, kv head) cache block, and the
 * new entry already rounded to `dtype` (k_hat, v_hat as dtype arrays). */
void orc_attend_block(double* o, const double* q_rot, const void* kc, const void* vc,
                      int dtype, int n, int D, const void* k_hat, const void* v_hat,
                      double scale, double ks, double vs)
{
    double* kn = (double*)malloc(sizeof(double) * (size_t)D);
    double* vn = (double*)malloc(sizeof(double) * (size_t)D);
    orc_decode(dtype, k_hat, (size_t)D, kn);
    orc_decode(dtype, v_hat, (size_t)D, vn);
    for (int d = 0; d < D; ++d) { kn[d] *= ks; vn[d] *= vs; }
    orc_attend(o, q_rot, kc, vc, dtype, n, D, kn, vn, scale, ks, vs);
    free(kn); free(vn);
}
