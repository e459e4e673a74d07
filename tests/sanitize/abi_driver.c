/* Sanitizer driver of the host side of libhswd (test infrastructure): the
 * library's sources built for the host only, with AddressSanitizer and
 * UndefinedBehaviorSanitizer, and every entry point called through its host
 * checks: null and misaligned pointers, bad descriptors, capacity errors,
 * empty batches, chunk and workspace sizing over the supported geometries
 * (caches up to 2^25 rows), and valid calls, which on a host without a GPU
 * must come back as HSWD_ERR_HIP.  Pointers are stand-ins and never
 * dereferenced on the host.  Exits 0 when every status is the expected one. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/hswd.h"
#include "../../include/hswd_measure.h"

static int fails = 0;
#define EXPECT(call, want) do { int32_t got_ = (int32_t)(call); if (got_ != (want)) { \
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
    ++fails; } } while (0)
#define EXPECT_NEG(call) do { int32_t got_ = (int32_t)(call); if (got_ >= 0) { \
    fprintf(stderr, "line %d: %s returned %d, expected an error\n", __LINE__, #call, got_); ++fails; } } while (0)

static void* const A = (void*)0x10000;       /* aligned stand-in */
static void* const M = (void*)0x10004;       /* misaligned for 16-byte tensors */

static hswd_attn_desc desc(int B, int H, int Hkv, int D, int S, int dt)
{
    hswd_attn_desc d = {B, H, Hkv, D, S, dt, 1.0f / sqrtf((float)D), 0, 0, NULL};
    return d;
}

int main(void)
{
    EXPECT(hswd_version() > 0, 1);
    for (int s = -7; s <= 1; ++s) if (!hswd_status_string(s)) ++fails;

    /* descriptor checks */
    hswd_attn_desc d = desc(2, 8, 8, 256, 511, HSWD_BF16);
    EXPECT(hswd_num_splits(NULL, 1, 0), HSWD_ERR_INVALID);
    hswd_attn_desc bad[] = {desc(-1, 8, 8, 256, 511, 2), desc(2, 0, 8, 256, 511, 2),
                            desc(2, 8, 3, 256, 511, 2), desc(2, 8, 8, 100, 511, 2),
                            desc(2, 8, 8, 256, 0, 2), desc(2, 8, 8, 256, 511, 9),
                            desc(2, 8, 8, 64, 511, HSWD_FP8_E4M3)};
    for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
        EXPECT_NEG(hswd_num_splits(&bad[i], 1, 0));
        EXPECT(hswd_workspace_bytes(&bad[i], 1, 0) == 0, 1);
        EXPECT_NEG(hswd_layer_step(A, A, A, A, A, A, A, A, 1, 256, 1e4, 0, &bad[i], A, 1 << 20, NULL));
    }
    hswd_attn_desc e = d;
    e.scale = NAN; EXPECT(hswd_num_splits(&e, 1, 0), HSWD_ERR_INVALID);
    e = d; e.keys_per_split = 100; EXPECT(hswd_num_splits(&e, 1, 0), HSWD_ERR_INVALID);
    e = d; e.chunks_per_workgroup = -1; EXPECT(hswd_num_splits(&e, 1, 0), HSWD_ERR_INVALID);

    /* chunk counts and workspace sizes over the supported geometries */
    const int dts[] = {HSWD_F32, HSWD_F16, HSWD_BF16, HSWD_FP8_E4M3};
    const int Ds[] = {64, 128, 256};
    const long Ss[] = {1, 2, 511, 4097, 131073, 1L << 20, (1L << 23) + 1, (1L << 25) - 1};
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 3; ++b)
            for (int c = 0; c < 8; ++c)
                for (int Hq = 8; Hq <= 64; Hq *= 2) {
                    hswd_attn_desc x = desc(3, Hq, 8, Ds[b], (int)Ss[c], dts[a]);
                    const int n = hswd_num_splits(&x, 0, (int)Ss[c] - 1);
                    if (dts[a] == HSWD_FP8_E4M3 && Ds[b] < 128) { EXPECT(n, HSWD_ERR_UNSUPPORTED); continue; }
                    if (n < 1 || n > 4096) { fprintf(stderr, "splits %d\n", n); ++fails; }
                    if (hswd_workspace_bytes(&x, 0, (int)Ss[c] - 1) == 0) ++fails;
                    if (hswd_workspace_bytes(&x, 1, 0) == 0) ++fails;
                }

    /* entry points: nulls, alignment, capacity, empty batch */
    EXPECT(hswd_ring_mask(NULL, NULL, A, 2, 511, 1, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_ring_mask(A, A, A, -1, 511, 1, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_ring_mask(NULL, NULL, NULL, 0, 511, 1, NULL), HSWD_OK);
    EXPECT(hswd_rope_apply(A, A, A, 2, 8, 8, 256, 255, 1e4, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_rope_apply(A, A, A, 2, 8, 8, 256, 256, -1.0, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_rope_apply(A, A, A, 2, 8, 8, 1 << 15, 64, 1e4, NULL), HSWD_ERR_UNSUPPORTED);
    EXPECT(hswd_rope_apply(NULL, NULL, NULL, 0, 8, 8, 256, 64, 1e4, NULL), HSWD_OK);
    EXPECT(hswd_kv_slot_write(M, A, A, A, A, &d, 1, NULL, A, NULL), HSWD_ERR_ALIGN);
    EXPECT(hswd_kv_slot_write(A, A, A, A, A, &d, 1, NULL, NULL, NULL), HSWD_ERR_WORKSPACE);
    EXPECT(hswd_decode_attn_sliding(A, A, A, A, NULL, A, A, &d, A, 1 << 20, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_decode_attn_sliding(A, M, A, A, A, A, A, &d, A, 1 << 20, NULL), HSWD_ERR_ALIGN);
    EXPECT(hswd_decode_attn_sliding(A, A, A, A, A, A, A, &d, A, 8, NULL), HSWD_ERR_WORKSPACE);
    hswd_attn_desc f = desc(2, 8, 8, 256, 4097, HSWD_BF16);
    EXPECT(hswd_decode_attn_full(A, A, A, A, A, A, A, 4097, &f, A, 1 << 24, NULL), HSWD_ERR_CAPACITY);
    EXPECT(hswd_decode_attn_full(A, A, A, A, A, A, A, -1, &f, A, 1 << 24, NULL), HSWD_ERR_INVALID);
    hswd_attn_desc z = desc(0, 8, 8, 256, 4097, HSWD_BF16);
    EXPECT(hswd_decode_attn_full(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 4096, &z, NULL, 0, NULL), HSWD_OK);
    EXPECT(hswd_layer_step(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 5e6, 4096, &z, NULL, 0, NULL), HSWD_OK);
    EXPECT(hswd_layer_step(A, A, A, A, A, A, A, A, 0, 63, 5e6, 4096, &f, A, 1 << 24, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_lse_merge(A, A, A, 2, 8, 256, 2000, NULL), HSWD_ERR_UNSUPPORTED);
    EXPECT(hswd_head_gate(NULL, A, A, 2, 8, 256, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_gate_proj(A, A, A, 2, 0, 8, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_measure_stream_read(A, 17, A, 8, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_measure_stream_read(A, 1 << 20, A, 0, NULL), HSWD_ERR_INVALID);
    EXPECT(hswd_measure_stream_read((void*)0x10008, 1 << 20, A, 8, NULL), HSWD_ERR_ALIGN);
    EXPECT(hswd_workspace_init(NULL, 64, NULL), HSWD_ERR_WORKSPACE);
    EXPECT(hswd_check_errors(NULL, NULL, NULL), HSWD_ERR_WORKSPACE);
    hswd_attn_desc g = desc(2, 16, 8, 256, 4097, HSWD_F32);       /* grouped f32: not built */
    EXPECT(hswd_layer_step(A, A, A, A, A, A, A, A, 0, 64, 5e6, 4096, &g, A, 1 << 24, NULL), HSWD_ERR_UNSUPPORTED);
    hswd_attn_desc big = desc(1, 8, 8, 256, (1 << 23) + 1, HSWD_F32);   /* 8 GiB block */
    EXPECT(hswd_layer_step(A, A, A, A, A, A, A, A, 0, 64, 5e6, 10, &big, A, 1 << 24, NULL), HSWD_ERR_UNSUPPORTED);

    /* the entry point that allocates nothing: refusals before any device work */
    hswd_attn_desc h64 = desc(2, 64, 8, 256, (1 << 20) + 1, HSWD_BF16);
    EXPECT(hswd_layer_step_noalloc(A, A, A, A, NULL, A, A, A, 0, 64, 5e6, 1 << 20, &h64, NULL, NULL), HSWD_ERR_WORKSPACE);
    hswd_attn_desc many = desc(2049, 8, 8, 256, 511, HSWD_BF16);
    EXPECT(hswd_layer_step_noalloc(A, A, A, A, NULL, A, A, A, 1, 256, 1e4, 0, &many, NULL, NULL), HSWD_ERR_WORKSPACE);
    EXPECT(hswd_layer_step_noalloc(A, A, A, A, NULL, A, A, A, 1, 256, 1e4, 0, &d, (int32_t*)0x10002, NULL), HSWD_ERR_ALIGN);

    /* valid calls: without a GPU they must fail in the HIP runtime, cleanly */
    EXPECT_NEG(hswd_layer_step(A, A, A, A, A, A, A, A, 1, 256, 1e4, 0, &d, A, 1 << 20, NULL));
    EXPECT_NEG(hswd_decode_attn_full(A, A, A, A, A, A, A, 4096, &f, A, 1 << 24, NULL));
    EXPECT_NEG(hswd_layer_step_noalloc(A, A, A, A, NULL, A, A, A, 1, 256, 1e4, 0, &d, NULL, NULL));

    if (fails) { fprintf(stderr, "%d checks failed\n", fails); return 1; }
    printf("abi sanitizer driver: ok\n");
    return 0;
}
