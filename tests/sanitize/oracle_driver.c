/* Sanitizer driver of the CPU oracle (test infrastructure): the oracle's
 * source compiled in with AddressSanitizer and UndefinedBehaviorSanitizer,
 * every public function called on small cases that reach its edges (every
 * cache type, rings below and past capacity, append caches at the capacity,
 * grouped heads, empty partials, odd sizes).  Exits 0 when every result is
 * finite where it must be; a sanitizer report aborts with a non-zero status. */
#include "../../oracle/hswd_oracle.c"

#include <stdio.h>

static unsigned rng_state = 12345u;
static float frand(void)                 /* uniform in [-2, 2) */
{
    rng_state = rng_state * 1664525u + 1013904223u;
    return (float)((rng_state >> 8) * (4.0 / 16777216.0) - 2.0);
}

static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static void one_step(int B, int H, int Hkv, int D, int n_slots, int dtype, int ring,
                     const int32_t* pos, int with_gate, int with_scale)
{
    int eb = elt_bytes(dtype);
    size_t ncache = (size_t)B * Hkv * n_slots * D, nq = (size_t)B * H * D, nkv = (size_t)B * Hkv * D;
    float* q = malloc(sizeof(float) * nq);
    float* k = malloc(sizeof(float) * nkv);
    float* v = malloc(sizeof(float) * nkv);
    float* g = malloc(sizeof(float) * (size_t)B * H);
    float* src = malloc(sizeof(float) * ncache);
    void* kc = malloc((size_t)eb * ncache);
    void* vc = malloc((size_t)eb * ncache);
    float sc[2 * 64];
    for (size_t i = 0; i < nq; ++i) q[i] = frand();
    for (size_t i = 0; i < nkv; ++i) { k[i] = frand(); v[i] = frand(); }
    for (int i = 0; i < B * H; ++i) g[i] = frand();
    for (int i = 0; i < 2 * Hkv; ++i) sc[i] = 0.01f + 0.003f * (float)i;
    for (size_t i = 0; i < ncache; ++i) src[i] = frand() * (with_scale ? 0.01f : 1.f);
    orc_round_f32_to(dtype, src, ncache, kc);
    for (size_t i = 0; i < ncache; ++i) src[i] = frand() * (with_scale ? 0.01f : 1.f);
    orc_round_f32_to(dtype, src, ncache, vc);
    double* out = malloc(sizeof(double) * nq);
    double* opre = malloc(sizeof(double) * nq);
    double* qr = malloc(sizeof(double) * nq);
    float* kr = malloc(sizeof(float) * nkv);
    void* kh = malloc((size_t)eb * nkv);
    void* vh = malloc((size_t)eb * nkv);
    int st = orc_layer_step(B, H, Hkv, D, n_slots, dtype, ring, ring ? D : D / 4,
                            ring ? 1e4 : 5e6, 1.0 / sqrt((double)D), 0, pos, q, k, v,
                            with_gate ? g : NULL, kc, vc, 1, with_scale ? sc : NULL,
                            out, opre, qr, kr, kh, vh);
    for (int b = 0; b < B; ++b) {
        int capacity_error = !ring && pos[b] >= n_slots;
        CHECK(!capacity_error || st == -4);
        for (int i = 0; i < H * D; ++i) CHECK(isfinite(out[(size_t)b * H * D + i]));
    }
    /* the per-(stream, head) entry of the full-size checks on the same data */
    for (int b = 0; b < B; ++b) {
        int p = pos[b], n = p < n_slots ? p : n_slots;
        for (int h = 0; h < H; ++h) {
            int gg = h / (H / Hkv);
            double o[512];
            size_t blk = ((size_t)b * Hkv + gg) * n_slots * D;
            orc_attend_block(o, qr + ((size_t)b * H + h) * D, (char*)kc + blk * eb,
                             (char*)vc + blk * eb, dtype, n, D,
                             (char*)kh + ((size_t)b * Hkv + gg) * D * eb,
                             (char*)vh + ((size_t)b * Hkv + gg) * D * eb, 1.0 / sqrt((double)D),
                             with_scale ? sc[gg] : 1.0, with_scale ? sc[Hkv + gg] : 1.0);
            for (int d = 0; d < D; ++d) CHECK(isfinite(o[d]));
        }
    }
    free(q); free(k); free(v); free(g); free(src); free(kc); free(vc);
    free(out); free(opre); free(qr); free(kr); free(kh); free(vh);
}

int main(void)
{
    /* element conversions at their edges */
    const float edge[] = {0.f, -0.f, 1.f, 65504.f, 65520.f, 1e-8f, -1e-40f, 3.4e38f, 448.f,
                          464.f, 1e6f, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof(edge) / sizeof(edge[0]); ++i) {
        (void)orc_f32_to_f16(edge[i]);
        (void)orc_f32_to_bf16(edge[i]);
        (void)orc_f32_to_fp8(edge[i]);
    }
    for (int c = 0; c < 256; ++c) (void)orc_fp8_value((uint8_t)c);
    for (int h = 0; h < 65536; ++h) { (void)orc_f16_value((uint16_t)h); (void)orc_bf16_value((uint16_t)h); }

    /* slot and mask */
    int32_t pos[6] = {0, 1, 510, 511, 512, 5000};
    int32_t slot[6];
    uint8_t mask[6 * 511];
    orc_slot_mask(6, 511, 1, pos, slot, mask);
    CHECK(mask[2 * 511 + 509] == 1 && mask[2 * 511 + 510] == 0 && slot[4] == 1);
    uint8_t* mask2 = malloc(6 * 5001);
    int32_t slot2[6];
    orc_slot_mask(6, 5001, 0, pos, slot2, mask2);
    CHECK(mask2[5 * 5001 + 4999] == 1 && mask2[5 * 5001 + 5000] == 0 && slot2[5] == 5000);
    free(mask2);

    /* layer steps: every cache type, ring and append, grouped heads */
    int32_t p_ring[4] = {0, 3, 7, 40};
    int32_t p_app[3] = {0, 5, 12};
    int32_t p_cap[2] = {12, 4};
    for (int dt = 0; dt < 4; ++dt) {
        int D = dt == 3 ? 128 : 64;
        one_step(4, 4, 4, D, 7, dt, 1, p_ring, 1, dt == 3);
        one_step(3, 8, 2, D, 13, dt, 0, p_app, 0, dt == 3);
        one_step(2, 4, 1, D, 12, dt, 0, p_cap, 1, dt == 3);   /* stream 0 at the capacity */
    }

    /* partials and merges, empty chunks included */
    {
        int D = 16, n = 9;
        float* src = malloc(sizeof(float) * n * D);
        uint16_t kc[9 * 16], vc[9 * 16];
        for (int i = 0; i < n * D; ++i) src[i] = frand();
        orc_round_f32_to(ORC_BF16, src, (size_t)n * D, kc);
        for (int i = 0; i < n * D; ++i) src[i] = frand();
        orc_round_f32_to(ORC_BF16, src, (size_t)n * D, vc);
        double q[16], kn[16], vn[16], o[16];
        for (int d = 0; d < D; ++d) { q[d] = frand(); kn[d] = frand(); vn[d] = frand(); }
        int32_t bounds[6] = {0, 0, 4, 4, 8, 9};
        orc_attend_split(o, q, kc, vc, ORC_BF16, bounds, 5, D, kn, vn, 0.25, 1.0, 1.0);
        for (int d = 0; d < D; ++d) CHECK(isfinite(o[d]));
        orc_attend(o, q, kc, vc, ORC_BF16, 0, D, kn, vn, 0.25, 1.0, 1.0);
        for (int d = 0; d < D; ++d) CHECK(o[d] == vn[d]);
        free(src);
    }

    /* gate projection and gate */
    {
        float x[3 * 100], w[7 * 100];
        double lg[21], og[3 * 7 * 5], oo[3 * 7 * 5];
        float gl[21];
        for (int i = 0; i < 300; ++i) x[i] = frand();
        for (int i = 0; i < 700; ++i) w[i] = frand();
        orc_gate_proj(lg, x, w, 3, 100, 7);
        for (int i = 0; i < 21; ++i) gl[i] = (float)lg[i];
        for (int i = 0; i < 105; ++i) oo[i] = frand();
        orc_head_gate(og, oo, gl, 3, 7, 5);
        CHECK(orc_sigmoid(0.0) == 0.5);
    }

    if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
