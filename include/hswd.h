/*
 * hswd.h -- hybrid sliding-window decode attention on AMD Instinct MI355X.
 *
 * C ABI of libhswd.so.  One decode step of one attention layer, for a batch
 * of B independent streams, each adding one token:
 *
 *   rotate q and k (RoPE, set per layer type)          hswd_rope_apply
 *   attend over the cached keys plus the new entry      hswd_decode_attn_sliding
 *     (ring of window-1 slots, or append cache),        hswd_decode_attn_full
 *     split over the key range and merged               hswd_lse_merge
 *   gate logits from the layer input (g_proj)           hswd_gate_proj
 *   scale each head by the sigmoid of its gate logit    hswd_head_gate
 *   store the new entry in its ring slot / append row   hswd_kv_slot_write
 *   all of the above in one launch                      hswd_layer_step,
 *                                                       hswd_layer_step_gproj
 *
 * Sources (web pages; each citation names the page and its part):
 *   [join]   vLLM-Omni fork commit log (tea.kyle-merritt.com,
 *            anodyine/vllm-omni), the commit that joins the new token to the
 *            cache in score space: scores of the cache and of the new token
 *            are joined as two vectors, no cache-sized tensor is copied, a
 *            ring needs no reordering, only a mask of unwritten slots, and it
 *            holds window-1 = 511 entries because the window counts the
 *            current token; each layer returns only the new K/V entry.
 *   [export] same log, the commit exporting one decode step with the caches
 *            sized per layer type (separate caches, masks, rotary angles)
 *            and moving the [2048, 8] head gate.
 *   [model]  same log, the commit adding the Spark-X2.5 model: three
 *            512-token sliding layers per full layer; sliding layers rotate
 *            all 256 head dims at theta 1e4, full layers the first quarter at
 *            theta 5e6; g_proj scales each head's output by a sigmoid.
 *   [talker] same log, the Qwen3-TTS talker decode-step commit: one cache
 *            tensor per layer, not one stacked tensor.
 *   [split]  TensorFold pull request 608 "Qwen3.8-27B on CUDA", review
 *            thread: split the key range of a long row so the GPU fills, and
 *            merge the partials; the split size is part of the summation
 *            order.
 *   [codec]  pega-omni pull request 4 "qwen3-tts: one kern manifest ...",
 *            codec attention commits: RoPE, ring write and attention in one
 *            launch per layer, window loads issued before the sync on q.
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers owned by the caller, unless stated.  The
 *     library never allocates, frees or synchronises, except in
 *     hswd_check_errors.  Every launch is asynchronous on `stream`
 *     (a hipStream_t; NULL is the null stream).
 *   - Tensors are dense, row-major, 16-byte aligned.  Shapes below use
 *     B streams, H query heads, Hkv kv heads (H % Hkv == 0), D = head_dim.
 *   - Caches are [B, Hkv, n_slots, D] of the cache element type, one buffer
 *     per layer [talker].  Ring: position t lives in slot t mod n_slots, and
 *     slots s >= min(pos, n_slots) are unwritten and never read.  Append:
 *     position t lives in row t, rows >= pos are never read.
 *   - pos[b] (int32, device) is the 0-based position of stream b's new
 *     token, i.e. the number of tokens before it.
 *   - Return value: HSWD_OK or a negative hswd_status.  Argument errors are
 *     found on the host before anything is launched.  A stream whose device
 *     pos is out of range sets a flag in the workspace's error word; read it
 *     with hswd_check_errors.
 *   - An empty batch (B = 0) is a no-op: once its other arguments pass, an
 *     entry returns HSWD_OK and launches nothing, whatever its pointers
 *     (an empty tensor may have none).  B < 0 is HSWD_ERR_INVALID.
 *   - Results are deterministic for a fixed keys_per_split and do not depend
 *     on B or on a stream's index in the batch.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef HSWD_H
#define HSWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Cache element types.  HSWD_FP8_E4M3 is OCP fp8 e4m3 (4 exponent bits,
 * bias 7, 3 fraction bits, no infinities, largest finite 448) with a scale
 * per kv head: a cached value is scale * decode(code); an entry x is stored
 * as the code of x / scale (the quotient rounded once to float32), rounded to
 * nearest even and saturated to +-448. */
typedef enum { HSWD_F32 = 0, HSWD_F16 = 1, HSWD_BF16 = 2, HSWD_FP8_E4M3 = 3 } hswd_dtype;

typedef enum {
    HSWD_OK = 0,
    HSWD_ERR_INVALID = -1,     /* bad size, null pointer or parameter */
    HSWD_ERR_ALIGN = -2,       /* a pointer is not 16-byte aligned */
    HSWD_ERR_WORKSPACE = -3,   /* workspace missing or too small */
    HSWD_ERR_CAPACITY = -4,    /* a position does not fit its cache */
    HSWD_ERR_HIP = -5,         /* a HIP runtime call failed */
    HSWD_ERR_UNSUPPORTED = -6  /* valid, but not built (head_dim, group) */
} hswd_status;

/* Bits of the workspace error word (hswd_check_errors). */
#define HSWD_FLAG_CAPACITY 1   /* append pos >= n_slots: write skipped */
#define HSWD_FLAG_MAX_POS 2    /* pos > max_pos: keys past max_pos unread */
#define HSWD_FLAG_NEG_POS 4    /* pos < 0 */

/* Shape and numerics of one attention layer. */
typedef struct {
    int32_t batch;          /* B >= 0 (0: an empty batch, nothing to do) */
    int32_t n_heads;        /* H */
    int32_t n_kv_heads;     /* Hkv, H % Hkv == 0.  Query head h reads kv head
                               h / (H / Hkv) (grouped-query attention by reshaping
                               the query [talker]); the attention entries take
                               H / Hkv = 1 with any cache, and any H / Hkv > 1
                               with a 16-bit or fp8 cache and head_dim 128 or 256
                               (else UNSUPPORTED).  Groups of 2 to 8 read the
                               cache once per layer (kernels for 2, 4 and 8
                               heads, a group below a kernel's size leaving
                               heads idle; 2 over an fp8 cache run the 4-head
                               kernel); a larger group is split into pieces
                               of eight query heads, one workgroup per piece in
                               the same launch, each reading the cache (the
                               last piece to finish writes the new entry). */
    int32_t head_dim;       /* D: 64, 128 or 256 (fp8 caches: 128 or 256) */
    int32_t n_slots;        /* ring: slots (window - 1, 511 [join]); append: capacity rows.
                               The attention entries take n_slots * head_dim *
                               element bytes < 4 GiB (one (stream, kv head)
                               block; else UNSUPPORTED). */
    int32_t kv_dtype;       /* hswd_dtype of the cache */
    float scale;            /* softmax scale, > 0; 1/sqrt(D) by convention */
    int32_t keys_per_split; /* keys per chunk, the unit of summation order [split]:
                               the valid keys are cut into chunks of this many,
                               each chunk's softmax partial is formed alone and
                               the partials are folded in chunk order.  0 =
                               library default.  Ring: from the slot count,
                               element type and head grouping: 2^floor(log2(
                               n_slots/32)) clamped to [128, 512], from 131072
                               slots on 2^floor(log2(n_slots/128)) up to 2048,
                               at least the floor F = 4 quanta (8 when n_heads >
                               n_kv_heads).  Append cache: each stream's own,
                               from its n = min(pos, max_pos) valid keys: the
                               smallest power of two >= max(F, ceil(n / 32)),
                               at most 1024 below n = 131072, 2048 below
                               n = 524288 and from there 1024 * n_kv_heads
                               within [2048, 8192] (so about 32 chunks of
                               them up to 32768 keys), then doubled while n
                               would need more than 4096 chunks.  Either way a function of the geometry
                               and the stream's own position, never of the
                               batch.
                               Else a multiple of the quantum Q = 32768 /
                               (head_dim * element bytes) keys (4 waves, one
                               8-load tile each): 64 for D = 256 and a 16-bit
                               cache, 32 for f32, 128 for fp8, that cuts the
                               key range into at most 4096 chunks (else
                               HSWD_ERR_INVALID).  Results depend on it; never
                               on the batch. */
    int32_t chunks_per_workgroup; /* work split only, never the bits: how many
                               consecutive chunks one workgroup streams.  0 =
                               library choice (from B and the CU count; for
                               append caches with max_pos >= 32768, at most 256
                               streams and at most 8 query heads per kv head,
                               dealt on the device from each stream's valid
                               keys: the fewest keys per workgroup whose
                               workgroups the GPU holds at once). */
    const float* kv_scale;  /* fp8 caches only: DEVICE pointer, float32 [2, Hkv],
                               the K scales then the V scales of the kv heads
                               (NULL = 1 for every head).  Ignored otherwise. */
} hswd_attn_desc;

/* Library version, (major << 16) | minor. */
int32_t hswd_version(void);

/* Human-readable name of a status code.  Static string; never NULL. */
const char* hswd_status_string(int32_t status);

/* Workspace bytes needed by the attention entries for this layer and the
 * largest position `max_pos` any stream will have (append caches; rings
 * ignore it).  The workspace holds the error word, the arrival counters (per
 * (stream, kv head) and head piece, and per (stream, kv head) for the entry
 * write of a group split into pieces) and the chunk partials.  It must be zeroed once before
 * first use (hswd_workspace_init); the library leaves the counters at zero
 * after every call, so it can be reused without clearing. */
size_t hswd_workspace_bytes(const hswd_attn_desc* d, int32_t ring, int32_t max_pos);

/* Zero a workspace (error word and counters) with a fill kernel. */
int32_t hswd_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Number of chunks per (stream, kv head) a launch is sized for (partials,
 * workspace): ceil(n_slots / K) for a ring, ceil(max_pos / K) for an append
 * cache with an explicit keys_per_split K, and under the append default the
 * most chunks any stream with pos <= max_pos can have: ceil(max_pos /
 * K(max_pos)), at least 32 once max_pos reaches 32 F, 4096 from 2^23 keys
 * (at least 1).  HSWD_ERR_INVALID (and a workspace size of 0) when that
 * exceeds 4096. */
int32_t hswd_num_splits(const hswd_attn_desc* d, int32_t ring, int32_t max_pos);

/* Slot and mask [join].  slot[b] = pos[b] mod n_slots (ring) or pos[b]
 * (append); mask[b][s] = 1 iff s < min(pos[b], n_slots), i.e. slot s holds a
 * token.  mask is uint8 [B, n_slots], slot int32 [B] (either may be NULL).
 * The decode kernels derive the same values internally; this entry exists
 * for inspection and bit-exact tests. */
int32_t hswd_ring_mask(uint8_t* mask, int32_t* slot, const int32_t* pos, int32_t B,
                       int32_t n_slots, int32_t ring, void* stream);

/* RoPE, in place [model].  q float32 [B, H, D], k float32 [B, Hkv, D] (k may
 * be NULL).  For i < rot_dim/2 the pair (x[i], x[i + rot_dim/2]) is rotated
 * by the angle pos[b] * theta^(-2i/rot_dim); dims >= rot_dim are unchanged.
 * Sliding layers: rot_dim = D, theta = 1e4; full layers: rot_dim = D/4,
 * theta = 5e6.  The angle, its sine and cosine and the rotation are computed
 * in double precision and rounded once to float32.  rot_dim even, 0 < rot_dim
 * <= D, theta > 0.  D above 16384 returns HSWD_ERR_UNSUPPORTED. */
int32_t hswd_rope_apply(float* q, float* k, const int32_t* pos, int32_t B, int32_t H,
                        int32_t Hkv, int32_t D, int32_t rot_dim, double theta,
                        void* stream);

/* Store the new entry [join].  k_rot, v float32 [B, Hkv, D] are rounded to the
 * cache element type (round to nearest, ties to even; NaN stays NaN) and
 * written to slot pos mod n_slots (ring) or row pos (append) of k_cache /
 * v_cache.  slot_out int32 [B] receives the row written (nullable; -1 for a
 * skipped stream).  ws: workspace whose error word records an append pos >=
 * n_slots (that stream is skipped) or pos < 0.  For a ring, call it after the
 * attention that reads the same cache: slot pos mod n_slots still holds
 * position pos - n_slots, which the new token attends. */
int32_t hswd_kv_slot_write(void* k_cache, void* v_cache, const float* k_rot, const float* v,
                           const int32_t* pos, const hswd_attn_desc* d, int32_t ring,
                           int32_t* slot_out, void* ws, void* stream);

/* Decode attention over a ring [join], [split].  o float32 [B, H, D] is the
 * attention output before the gate:
 *   softmax over { scale * q_rot . K[s] : s < min(pos, n_slots) }
 *           joined with { scale * q_rot . k_hat },
 *   o = sum of weights * values (V[s] and v_hat) / sum of weights,
 * where k_hat, v_hat are k_rot, v rounded to the cache element type (the
 * entry hswd_kv_slot_write stores).  The ring is not modified.  Requires
 * H == Hkv.  ws: hswd_workspace_bytes(d, 1, 0) bytes. */
int32_t hswd_decode_attn_sliding(float* o, const float* q_rot, const float* k_rot,
                                 const float* v, const void* k_ring, const void* v_ring,
                                 const int32_t* pos, const hswd_attn_desc* d, void* ws,
                                 size_t ws_bytes, void* stream);

/* Decode attention over an append cache [join], [split]: as above over rows
 * 0..pos-1.  max_pos (host) bounds every pos[b] and sizes the split grid;
 * max_pos + 1 <= n_slots.  A larger device pos sets HSWD_FLAG_MAX_POS and
 * only keys below the grid's end are read. */
int32_t hswd_decode_attn_full(float* o, const float* q_rot, const float* k_rot,
                              const float* v, const void* k_cache, const void* v_cache,
                              const int32_t* pos, int32_t max_pos, const hswd_attn_desc* d,
                              void* ws, size_t ws_bytes, void* stream);

/* Chunk partials of the cached keys alone (no new entry) [split]: for chunk
 * c covering cache rows [c*K, (c+1)*K) of the valid range (K the stream's
 * chunk: keys_per_split, or the default of the descriptor's comment; chunks
 * past the stream's valid keys are empty),
 *   part_ml[b][h][c] = (m, l): m = max scale*q.K (natural-log units, -inf if
 *                      the split is empty), l = sum exp(score - m) (0 if empty);
 *   part_o[b][h][c][:] = sum exp(score - m) * V  (not divided by l).
 * part_o float32 [B, H, n, D], part_ml float32 [B, H, n, 2], with
 * n = hswd_num_splits(d, ring, max_pos). */
int32_t hswd_decode_attn_partials(float* part_o, float* part_ml, const float* q_rot,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* pos, int32_t ring, int32_t max_pos,
                                  const hswd_attn_desc* d, void* stream);

/* Log-sum-exp merge of n partials [split] (n <= 1024):
 *   M = max m_i over partials with l_i > 0,
 *   o[b][h][:] = sum part_o_i * exp(m_i - M) / sum l_i * exp(m_i - M).
 * Partials with l_i == 0 are skipped; at least one must be non-empty. */
int32_t hswd_lse_merge(float* o, const float* part_o, const float* part_ml, int32_t B,
                       int32_t H, int32_t D, int32_t n, void* stream);

/* Head gate [model], [export]: out[b][h][:] = o[b][h][:] / (1 + exp(-gate[b][h])).
 * gate float32 [B, H] are g_proj's logits.  out may alias o. */
int32_t hswd_head_gate(float* out, const float* o, const float* gate, int32_t B, int32_t H,
                       int32_t D, void* stream);

/* One whole layer step in one launch [codec], [join]: rotate q and k (from
 * the unrotated float32 q [B,H,D], k [B,Hkv,D]), attend as
 * hswd_decode_attn_sliding (ring != 0) or hswd_decode_attn_full (ring == 0),
 * gate (gate may be NULL: no gate), write the gated output to out [B,H,D],
 * then store the rounded entry in the cache.  The store is ordered after
 * every read of that (stream, kv head)'s cache within the launch.  Same
 * numbers as the four separate entries.  q, k and v are not modified. */
int32_t hswd_layer_step(float* out, const float* q, const float* k, const float* v,
                        const float* gate, void* k_cache, void* v_cache, const int32_t* pos,
                        int32_t ring, int32_t rot_dim, double theta, int32_t max_pos,
                        const hswd_attn_desc* d, void* ws, size_t ws_bytes, void* stream);

/* hswd_layer_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same kernels and the same numbers as
 * hswd_layer_step; the workspace is a device array the library owns, one
 * per GPU, HSWD_NOALLOC_SCRATCH_BYTES (32 MiB) each, held until the process
 * ends.  Nothing is allocated or freed: the first call on a GPU looks up the
 * array's address and clears it with a fill kernel on `stream` (captured
 * with the call if that first call is under capture).
 *   err: DEVICE int32 (4-byte aligned, nullable) into which the HSWD_FLAG_*
 *        bits are OR-ed (read them with hswd_check_errors(err, ...)); when
 *        NULL they are recorded in the array and cannot be read.
 * Returns HSWD_ERR_WORKSPACE, before touching the device, when the call
 * would need more than the array holds: 64 KiB of arrival counters (B * Hkv
 * per head piece, plus B * Hkv when a group is split into pieces) and the
 * chunk partials B * H * n_chunk * (D + 2) * 4 bytes, needed only when the
 * work split puts a (stream, kv head) on several workgroups (long contexts,
 * small batches).  Every call on one GPU shares its array, whose arrival
 * counters each call leaves at zero: calls that overlap in time on one GPU
 * (several streams or host threads) race and must be serialised. */
#define HSWD_NOALLOC_SCRATCH_BYTES (32u << 20)
int32_t hswd_layer_step_noalloc(float* out, const float* q, const float* k, const float* v,
                                const float* gate, void* k_cache, void* v_cache,
                                const int32_t* pos, int32_t ring, int32_t rot_dim, double theta,
                                int32_t max_pos, const hswd_attn_desc* d, int32_t* err,
                                void* stream);

/* Gate projection g_proj [model], [export]: logits[b][h] = sum over i of
 * x[b][i] * w_g[h][i], summed in a fixed order in float32.  x float32
 * [B, hidden] is the layer's post-norm input (the same one the QKV
 * projection reads); w_g float32 [H, hidden] is the projection's weight in
 * the row-per-output layout of a linear layer (the pages' model maps hidden
 * 2048 to 8 heads; each head's row is contiguous).  logits float32 [B, H]. */
int32_t hswd_gate_proj(float* logits, const float* x, const float* w_g, int32_t B,
                       int32_t hidden, int32_t H, void* stream);

/* hswd_layer_step with the gate logits computed inside the launch from x
 * [B, hidden] and w_g [H, hidden] (the same sum as hswd_gate_proj, so the
 * same bits as hswd_gate_proj followed by hswd_layer_step). */
int32_t hswd_layer_step_gproj(float* out, const float* q, const float* k, const float* v,
                              const float* x, const float* w_g, int32_t hidden, void* k_cache,
                              void* v_cache, const int32_t* pos, int32_t ring, int32_t rot_dim,
                              double theta, int32_t max_pos, const hswd_attn_desc* d, void* ws,
                              size_t ws_bytes, void* stream);

/* Synchronise `stream`, then read the workspace error word.  Returns
 * HSWD_OK if it is zero, HSWD_ERR_CAPACITY otherwise; *flags_out (nullable,
 * host) receives the HSWD_FLAG_* bits.  Flags stay set until
 * hswd_workspace_init. */
int32_t hswd_check_errors(const void* ws, int32_t* flags_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSWD_H */
