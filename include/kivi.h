/*
 * kivi.h -- C ABI of libkivi: a 2-bit KIVI KV cache and fused decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (pages on KIVI, cited by title and section):
 *  - "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache" (arXiv 2402.02750v2
 *    summary): title ("asymmetric 2bit"); "Key points"/"Summary": serving batches many
 *    requests and the KV cache becomes the speed and memory bottleneck as batch and
 *    context grow, so the cache is quantized.
 *  - inference-research record kv-efficiency/kivi-2bit-llama2-13b-mha-4k, "KV bytes
 *    basis", "Quant method" and "Methodology": keys quantized per-channel and values
 *    per-token, group size 32, the most recent R = 128 tokens kept in 16-bit floats and
 *    only the grouped history quantized.
 *  - "Your KV cache doesn't have a bit problem, it has a geometry problem", paragraphs
 *    1-4: why keys go per-channel (fixed outlier channels) and values per-token (errors
 *    matter at the attention output), and the full-precision residual.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked (host).  The caller allocates and frees
 *    every buffer; the library allocates nothing, on any path.  Its only mutable global
 *    state is the per-device scratch of kivi_decode_attn_noalloc (static device memory of
 *    the library) and the per-thread settings of the measurement and testing hooks.  fp16
 *    data are IEEE binary16 bit patterns (uint16_t).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work on
 *    it and never synchronise the device.
 *  - Return value: KIVI_OK (0) or a negative KIVI_ERR_* code.  Arguments are validated
 *    on the host before anything is enqueued; on any error nothing is enqueued and the
 *    cache state fields are unchanged.  Nothing throws across this boundary.
 *  - Inputs must be finite (NaN/Inf are outside the contract and are not scanned).
 *  - This version implements head_dim == 128 and group 32, 64 or 128 (other valid shapes
 *    return KIVI_ERR_UNSUPPORTED).  The pages' configuration is G = 32, R = 128; G and R
 *    are parameters of the descriptor.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KIVI_OK = 0,
    KIVI_ERR_NULL = -1,          /* a required pointer is NULL */
    KIVI_ERR_SHAPE = -2,         /* sizes inconsistent (divisibility, empty context, ...) */
    KIVI_ERR_UNSUPPORTED = -3,   /* valid but not implemented here (head_dim != 128, ...) */
    KIVI_ERR_CAPACITY = -4,      /* the call would write past token_cap / residual_cap */
    KIVI_ERR_WORKSPACE = -5,     /* workspace missing or too small */
    KIVI_ERR_HIP = -6,           /* a HIP runtime error while enqueueing */
    KIVI_ERR_STATE = -7          /* the cache state fields are inconsistent */
};

/*
 * The cache descriptor (host struct; the caller owns it and every buffer it points to).
 * row = b * kv_heads + h.  D = head_dim, G = group, R = residual_cap.
 *
 * Packed layout (four 2-bit codes per byte; D = 128).  The codes are stored in tiles of
 * 32 tokens whatever G is (a key group of G tokens spans G/32 tiles):
 *   k_codes, v_codes : uint8  [row][token_cap/32][1024]: one 1024-byte tile per 32 tokens.
 *                      k_codes: a little-endian 32-bit word holds channels 16w..16w+15 of
 *                        one token, channel 16w + 4i + b in byte b at bits 2i..2i+1, so
 *                        masking a word with 0x03030303 << 2i yields the codes of four
 *                        consecutive channels, one per byte; 16-byte chunk (16k + n) of a
 *                        tile holds words k and 4+k of its token n, then words k and 4+k of
 *                        its token 16+n (k = 0..3, n = 0..15).
 *                      v_codes: a byte holds one channel's codes for four consecutive
 *                        tokens, token 4a+i at bits 2i..2i+1; 16-byte chunk (16k + n) of a
 *                        tile covers its tokens 8k..8k+7, and the chunk's byte 4p + 2h + e
 *                        holds channel n + 16(2p + e) for tokens 8k+4h..8k+4h+3 (k = 0..3,
 *                        n = 0..15, p = 0..3, h and e = 0..1).
 *   (KIVI_CODES_4BIT)  k_codes, v_codes : uint8 [row][token_cap][D/2] instead: a token's
 *                      codes in D/2 bytes, channel j in byte j/2, the even channel in the
 *                      low nibble.  A 4-bit cache holds at most 2^26 tokens a row
 *                      (token_cap above that: KIVI_ERR_UNSUPPORTED).
 *   k_sz             : fp16   [row][token_cap/G][D][2]  (scale, zero) of key token group
 *                      g (tokens Gg..Gg+G-1), channel j -- keys are quantized per-channel
 *                      over G tokens.
 *   v_sz             : fp16   [row][token_cap][D/G][2]  (scale, zero) of value token t,
 *                      channel group k (channels Gk..Gk+G-1) -- values are quantized
 *                      per-token over G channels.
 *   k_res, v_res     : fp16   [row][R][D] residual ring; the n_res newest tokens, oldest
 *                      first, sit in slots (res_head + i) % R, i < n_res.
 * Dequantized value: zero + code * scale.  Quantizer: zero = group min, scale =
 * fp16(fp32(fp32(max - min) / 3)), code = clamp(round_half_even(fp32(fp32(x - min) /
 * scale)), 0, 3) (scale 0 -> code 0), a -0 minimum stored as +0.
 *
 * State: the first n_quant tokens of the context (a multiple of G) are in the quantized
 * history; the next n_res (0..R) are in the ring.  res_head is a multiple of G.
 */
/* Flush policy (kivi_cache.flags).  Default (0): a full residual gives its oldest G tokens
 * to the history when a token arrives.  KIVI_FLUSH_ALL: it gives all R of them (R/G groups),
 * the other reading of the residual length of the pages' ablation (summary page, "Key
 * points"): the full-precision buffer fills up to R and is then quantized as a whole. */
#define KIVI_FLUSH_ALL 1
/* Code width (kivi_cache.flags).  Default (0): 2-bit codes, four levels (KIVI-2, the
 * summary page's and the record's scheme).  KIVI_CODES_4BIT: 4-bit codes, sixteen levels
 * with the same rules (scale = (max - min)/15, codes clamped at 15), in the layout below. */
#define KIVI_CODES_4BIT 2

typedef struct kivi_cache {
    int32_t batch, kv_heads, head_dim;
    int32_t group;           /* G */
    int32_t residual_cap;    /* R, a multiple of G */
    int32_t token_cap;       /* capacity of the quantized history in tokens, multiple of G */
    int32_t n_quant, n_res, res_head;
    int32_t flags;           /* 0, or KIVI_FLUSH_ALL and/or KIVI_CODES_4BIT */
    uint8_t* k_codes;
    uint8_t* v_codes;
    uint16_t* k_sz;
    uint16_t* v_sz;
    uint16_t* k_res;
    uint16_t* v_res;
} kivi_cache;

/* Keys per-channel (record "Quant method"; article paragraph 2).
 * k: fp16, element (row, t, j) at k[row*src_row_stride + t*D + j], t < tokens.
 * Quantizes token groups [0, tokens) into history tokens [dst_token_off, +tokens).
 * tokens and dst_token_off are multiples of G; src_row_stride >= tokens*D.
 * Does not read or change the state fields. */
int kivi_quantize_k_per_channel(const uint16_t* k, int32_t tokens, int64_t src_row_stride,
                                kivi_cache* cache, int32_t dst_token_off, void* stream);

/* Values per-token (record "Quant method"; article paragraph 3): every token's D
 * channels in D/G groups of G.  Same source convention; any tokens >= 0 and any
 * dst_token_off >= 0 with dst_token_off + tokens <= token_cap. */
int kivi_quantize_v_per_token(const uint16_t* v, int32_t tokens, int64_t src_row_stride,
                              kivi_cache* cache, int32_t dst_token_off, void* stream);

/* Prefill from a context of `tokens` fp16 keys and values (same source convention):
 * quantizes the first n_quant (multiple of G, <= token_cap) tokens of both, copies the
 * remaining tokens - n_quant (<= R) into ring slots 0.. and sets n_quant, n_res and
 * res_head = 0 in *cache (host side, immediately). */
int kivi_prefill(const uint16_t* k, const uint16_t* v, int32_t tokens, int64_t src_row_stride,
                 int32_t n_quant, kivi_cache* cache, void* stream);

/* One decode-time token per row (k_new, v_new: fp16 [row][D], contiguous).
 * The record keeps the newest R tokens in 16-bit floats and quantizes only grouped
 * history ("KV bytes basis").  If the ring already holds R tokens, the oldest F of them
 * (F = G, or R with KIVI_FLUSH_ALL) become key token groups n_quant/G.. and value tokens
 * n_quant..n_quant+F-1 (flush), then the new token enters the ring.  Updates n_quant, n_res and res_head on the host
 * immediately (no device round trip).  *flushed (host, nullable) receives 1 if a group
 * was flushed, else 0.  KIVI_ERR_CAPACITY if a flush would pass token_cap. */
int kivi_append_flush(kivi_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                      int32_t* flushed, void* stream);

/* Fused decode attention over the whole cache, one query per head: the quantized history,
 * dequantized (zero + code * scale), followed by the fp16 residual ring, oldest first (record
 * "KV bytes basis": the grouped history quantized and the newest tokens kept in 16-bit
 * floats; the 2-bit bytes counted per token are what this call streams), with the error
 * judged at this output ("Your KV cache doesn't have a bit problem...", paragraph 3):
 * out = softmax(sm_scale * q.K^T) . V.
 * q: fp16 [batch][q_heads][D]; q_heads a multiple of kv_heads, query head hq reads kv
 * head hq / (q_heads / kv_heads).  out: fp16 [batch][q_heads][D].  lse (nullable): fp32
 * [batch][q_heads], natural log of the softmax denominator including sm_scale.
 * The context is split into num_splits parts per row (0 = automatic) and the partial
 * softmax states are merged with a log-sum-exp merge inside the same kernel launch.
 *
 * workspace: device scratch of at least kivi_decode_attn_workspace(cache, q_heads,
 * num_splits) bytes, 256-byte aligned, owned by the caller.  The whole workspace must be
 * zero before the first call that uses it (clear it once after allocating it); calls keep
 * it consistent afterwards.  Layout: a 32-bit status word at byte 0 (in a 256-byte block),
 * then a per-query-row arrival counter (zero again after every completed call) and a
 * per-query-row call epoch (round_up(8*batch*q_heads, 256) bytes), then the split partials,
 * each value stored with its call's tag.  The tag of a call's partials for a group of query
 * rows is one more than the largest epoch of those rows, and the merge sets each row's epoch
 * to it, so every attention entry point of this header (plain, pre-RoPE, ragged, fused step,
 * 2- or 4-bit) may use one workspace in any order for caches of one (batch, q_heads) shape;
 * clear it again before using it for another shape.  Calls that share a workspace must not run
 * concurrently.  Status word: the kernels OR in KIVI_WS_POLL_TIMEOUT when a merge gave up
 * waiting for a split partial (the merge polls each value a bounded number of times); the
 * rows concerned get out = NaN and lse = NaN.  The library never clears the word.  The next
 * word of the block holds the work share the last ragged call planned with, where the next
 * ragged call starts its search (any value there is safe: the plan checks it).
 * KIVI_ERR_SHAPE if the context is empty. */
#define KIVI_WS_POLL_TIMEOUT 1
int kivi_decode_attn(const kivi_cache* cache, const uint16_t* q, int32_t q_heads,
                     float sm_scale, uint16_t* out, float* lse, void* workspace,
                     size_t workspace_bytes, int32_t num_splits, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): kivi_decode_attn with the library's own scratch in
 * place of the caller's workspace.  Same arguments (minus workspace and workspace_bytes),
 * results, kernels, split count and errors as kivi_decode_attn; the caller still passes q,
 * out and lse.  The scratch is KIVI_NOALLOC_SCRATCH_BYTES of static device memory per device,
 * held until the process ends; a call whose kivi_decode_attn_workspace(cache, q_heads,
 * num_splits) exceeds it returns KIVI_ERR_WORKSPACE.  The call uses the scratch of the device
 * current on the calling thread (its first call there takes the scratch's address and clears
 * it on `stream`); it allocates nothing and calls no allocating routine.  Every call on one
 * device shares that scratch and leaves its contents for the next: calls of one (batch,
 * q_heads) shape keep it consistent as a workspace is kept, and a call of another shape first
 * clears what earlier calls used (one small kernel on `stream`).  Calls that overlap on one
 * device (other threads, other streams) race on the scratch: the caller serialises them.  The
 * scratch's status word (see kivi_decode_attn) is not readable from the host. */
#define KIVI_NOALLOC_SCRATCH_BYTES (8u << 20)
int kivi_decode_attn_noalloc(const kivi_cache* cache, const uint16_t* q, int32_t q_heads, float sm_scale,
                             uint16_t* out, float* lse, int32_t num_splits, void* stream);

/* Decode attention over a cache of pre-RoPE keys ("Your KV cache doesn't have a bit
 * problem...", paragraph 4, and the KVQuant summary on GrooveSquid advise quantizing keys
 * before the rotary position embedding; keys are then stored and appended as given, and the
 * rotation happens here, after dequantization).  Same arguments, results, workspace and
 * error behaviour as kivi_decode_attn, plus rope_base (> 0, finite; 10000 for Llama-2):
 * every key -- history token t at position t, the i-th oldest residual token at
 * n_quant + i -- is turned by the rotary embedding in rotate-half form (channel i < D/2
 * with channel i + D/2, angle position * rope_base^(-2i/D)) before q . k.  q is used as
 * given: the caller rotates it at its own position.  Values are not rotated.  The split
 * count for num_splits == 0 is kivi_decode_attn_rope_splits(); size the workspace with
 * kivi_decode_attn_workspace(cache, q_heads, that count).  2-bit caches take token_cap
 * <= 2^27 here (KIVI_ERR_UNSUPPORTED beyond).  One query head per workgroup.  The fused form
 * with the append is kivi_decode_step_rope. */
int kivi_decode_attn_rope(const kivi_cache* cache, const uint16_t* q, int32_t q_heads, float sm_scale,
                          float rope_base, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                          int32_t num_splits, void* stream);

/* kivi_decode_attn_rope for a ragged batch (per-sequence states as for
 * kivi_decode_attn_ragged): each sequence's keys are turned at that sequence's own positions
 * (history token t at t, the i-th oldest residual token at its n_quant + i).  num_splits == 0:
 * kivi_decode_attn_rope_ragged_splits; size the workspace with kivi_decode_attn_workspace(cache,
 * q_heads, that count).  A sequence with an empty context gets out = 0 and lse = -inf; a
 * state out of range is skipped and flagged KIVI_SEQ_BAD_STATE. */
int kivi_decode_attn_rope_ragged(const kivi_cache* cache, int32_t* seq_state, const uint16_t* q, int32_t q_heads,
                                 float sm_scale, float rope_base, uint16_t* out, float* lse, void* workspace,
                                 size_t workspace_bytes, int32_t num_splits, void* stream);

/* One whole decode step: kivi_append_flush(cache, k_new, v_new, flushed, stream) followed by
 * kivi_decode_attn(cache, q, ...) on the updated cache, with the same arguments, results,
 * state update and errors as those two calls (record "KV bytes basis": the newest R tokens
 * in 16-bit floats; decoding attends over the history and the residual, the new token
 * included).  When the ring has room it is one kernel launch: attention reads the new
 * token straight from k_new / v_new while one workgroup per KV head writes it into its
 * ring slot; when a group must be flushed first it is the two launches of the separate
 * calls.  The workspace must fit the attention on the state after the append: when the
 * ring is full that is kivi_decode_attn_workspace of the cache with n_quant + F.
 * Validation happens before anything is enqueued, so on error nothing changes. */
int kivi_decode_step(kivi_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                     const uint16_t* q, int32_t q_heads, float sm_scale, uint16_t* out, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t num_splits, int32_t* flushed,
                     void* stream);

/* kivi_decode_step with pre-RoPE attention: kivi_append_flush(cache, k_new, v_new, flushed,
 * stream) (the new key pre-RoPE, as stored) followed by kivi_decode_attn_rope(cache, q, ...)
 * on the updated cache, the new token at position n_quant + n_res - 1 of the updated state;
 * the same arguments, results, state update and errors as those two calls, one kernel
 * launch when no group is flushed (as in kivi_decode_step).  num_splits == 0 takes
 * kivi_decode_attn_rope_splits() of the updated state; the workspace must fit that count. */
int kivi_decode_step_rope(kivi_cache* cache, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                          int32_t q_heads, float sm_scale, float rope_base, uint16_t* out, float* lse,
                          void* workspace, size_t workspace_bytes, int32_t num_splits, int32_t* flushed,
                          void* stream);

/* ---- Ragged batches: sequences of one batch at different lengths.
 * The per-sequence cache state lives in device memory, seq_state: int32 [batch][4] =
 * {n_quant, n_res, res_head, flags}, 16-byte aligned, owned by the caller; the first three
 * mean for sequence b (rows b*kv_heads .. b*kv_heads + kv_heads - 1) what the kivi_cache
 * fields of the same names mean for a whole batch, and the descriptor's own n_quant, n_res
 * and res_head are ignored by these calls.  A sequence's rows are contiguous in every
 * buffer, so each sequence can be filled by the single-batch calls (kivi_prefill, ...) on
 * a descriptor with batch = 1 whose pointers start at its first row.  The kernels check
 * each state: one out of range (n_quant not a multiple of G or above token_cap, n_res
 * above residual_cap, res_head not a multiple of G below residual_cap) is not used, the
 * sequence attends over nothing and its flags get KIVI_SEQ_BAD_STATE.  flags bits are only
 * ever set (OR) by the library, never cleared. */
#define KIVI_SEQ_CAPACITY 1    /* an append was skipped: its flush would pass token_cap */
#define KIVI_SEQ_BAD_STATE 2   /* the sequence's state was out of range and was not used */

/* kivi_append_flush for every sequence of a ragged batch: one new token per sequence
 * (k_new, v_new: fp16 [batch][kv_heads][128]), a sequence whose ring is full first
 * flushing its oldest F ring tokens into new groups, then each sequence's state moved on
 * on the device (two kernel launches in stream order).  A sequence whose flush would pass
 * token_cap is left as it was and gets KIVI_SEQ_CAPACITY. */
int kivi_append_flush_ragged(const kivi_cache* cache, int32_t* seq_state, const uint16_t* k_new,
                             const uint16_t* v_new, void* stream);

/* kivi_decode_attn for a ragged batch: each sequence's query heads attend over that
 * sequence's history and residual.  The grid is sized for the longest context the cache can
 * hold (num_splits == 0: kivi_decode_attn_ragged_splits; the workspace is
 * kivi_decode_attn_workspace(cache, q_heads, that split count)); each workgroup finds its
 * sequence's share on the device.  A sequence with an empty context gets out = 0 and
 * lse = -inf. */
int kivi_decode_attn_ragged(const kivi_cache* cache, int32_t* seq_state, const uint16_t* q,
                            int32_t q_heads, float sm_scale, uint16_t* out, float* lse,
                            void* workspace, size_t workspace_bytes, int32_t num_splits, void* stream);

/* fp16 comparator (a measurement baseline, not the method): decode attention of one query
 * per head over a plain fp16 KV cache, the uncompressed cache the pages set the 2-bit
 * cache against (record "KV bytes basis": the 16-bit cache's bytes per token; "Methodology":
 * the throughput claim against the 16-bit baseline), on the same harness: same query
 * grouping, split-K and merge as kivi_decode_attn.
 * k, v: fp16 [batch][kv_heads][token_stride][128], tokens [0, tokens) of each row used,
 * 16-byte aligned, owned by the caller.  q, out, lse, workspace (at least
 * kivi_decode_attn_fp16_workspace(...) bytes, 256-byte aligned, zero before its first use,
 * the same layout as kivi_decode_attn's), num_splits (0 = automatic) and stream as in
 * kivi_decode_attn.  KIVI_ERR_SHAPE if tokens < 1, tokens > token_stride, q_heads is not a
 * multiple of kv_heads or a pointer is misaligned. */
int kivi_decode_attn_fp16(const uint16_t* k, const uint16_t* v, int32_t batch, int32_t kv_heads,
                          int32_t tokens, int32_t token_stride, const uint16_t* q, int32_t q_heads,
                          float sm_scale, uint16_t* out, float* lse, void* workspace,
                          size_t workspace_bytes, int32_t num_splits, void* stream);

/* Measurement hook, for callers that time the attention kernel itself (not a step of the
 * method).  The next decode-attention kernel that an attention call (kivi_decode_attn,
 * kivi_decode_step and the other attention entry points) or a read probe launches from
 * the calling thread records its own start in start_event and its end in
 * stop_event (hipEvent_t handles, created by the caller with timing enabled), taken by the
 * dispatch itself with no marker command in the stream, so hipEventElapsedTime(start, stop)
 * is that kernel's duration.  The setting is consumed by that one launch (a flush kernel
 * launched before it by kivi_decode_step is not timed); both NULL clears it.
 * KIVI_ERR_NULL if exactly one of the two is NULL.  No device access. */
int kivi_time_next_attention(void* start_event, void* stop_event);

/* Measurement helper (not a step of the method): reads `bytes` (a multiple of 16) of device
 * memory at src (16-byte aligned) once, in a plain grid-stride sweep of 16-byte loads, and
 * writes one word per workgroup to sink (device, at least kivi_read_probe_sink_bytes() bytes)
 * so that the loads are kept.  Timed, it gives the chip's streaming-read rate, the ceiling
 * beside the published HBM peak; untimed over more than the 256 MB Infinity Cache, it evicts
 * a working set from that cache between timed launches.  KIVI_ERR_NULL / KIVI_ERR_SHAPE on
 * bad arguments; nothing is enqueued then. */
int kivi_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);
size_t kivi_read_probe_sink_bytes(void);

/* kivi_read_probe with non-temporal loads (the hint the decode kernels stream the cache with):
 * the fastest plain read measured, so its rate is the read ceiling; it does not evict the
 * Infinity Cache.  Same arguments, errors and timing hook as kivi_read_probe. */
int kivi_read_probe_stream(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Testing hook of the merge's bounded wait (not a step of the method): the next attention call
 * of the calling thread that passes validation polls each split partial at most max_polls
 * times (0 = the library's bound) and waits for the tag tag_skew above its own (0 = its own).
 * With tag_skew != 0 no partial ever matches, so a multi-split call takes the give-up path
 * (NaN rows, KIVI_WS_POLL_TIMEOUT) after max_polls short sleeps per value, and every kernel
 * still ends.  KIVI_ERR_SHAPE if max_polls < 0.  No device access. */
int kivi_test_next_attention_merge(int32_t max_polls, uint32_t tag_skew);

/* Host-only helpers (no device access; safe without a GPU). */

/* Split count that kivi_decode_attn uses for num_splits == 0 (depends on shapes only).
 * Returns a value >= 1, or a negative KIVI_ERR_* code. */
int32_t kivi_decode_attn_splits(const kivi_cache* cache, int32_t q_heads);

/* Workspace bytes kivi_decode_attn needs for this shape and split count (0 = auto). */
size_t kivi_decode_attn_workspace(const kivi_cache* cache, int32_t q_heads, int32_t num_splits);

/* Split count that kivi_decode_step (pre_rope == 0) or kivi_decode_step_rope (pre_rope != 0)
 * uses for num_splits == 0: the attention's choice on the state after the step's append
 * (record "KV bytes basis": a full ring first gives its oldest tokens to the grouped history,
 * which lengthens it).  A negative KIVI_ERR_* code for an invalid shape or state, or
 * KIVI_ERR_CAPACITY if that append would pass token_cap. */
int32_t kivi_decode_step_splits(const kivi_cache* cache, int32_t q_heads, int32_t pre_rope);

/* Workspace bytes that kivi_decode_step / kivi_decode_step_rope (pre_rope != 0) needs with
 * num_splits (0 = kivi_decode_step_splits): kivi_decode_attn_workspace of the state after the
 * append.  0 for an invalid shape or state, or an append past token_cap. */
size_t kivi_decode_step_workspace(const kivi_cache* cache, int32_t q_heads, int32_t num_splits, int32_t pre_rope);

/* Split count kivi_decode_attn_rope uses for num_splits == 0 (depends on shapes only);
 * a negative KIVI_ERR_* code for an invalid shape or state. */
int32_t kivi_decode_attn_rope_splits(const kivi_cache* cache, int32_t q_heads);

/* Split count kivi_decode_attn_rope_ragged uses for num_splits == 0 (shape only). */
int32_t kivi_decode_attn_rope_ragged_splits(const kivi_cache* cache, int32_t q_heads);

/* Split count kivi_decode_attn_ragged uses for num_splits == 0 (shape only). */
int32_t kivi_decode_attn_ragged_splits(const kivi_cache* cache, int32_t q_heads);

/* Split count and workspace bytes of kivi_decode_attn_fp16 for this shape (0 = auto
 * splits); a negative KIVI_ERR_* code / 0 for an invalid shape. */
int32_t kivi_decode_attn_fp16_splits(int32_t batch, int32_t kv_heads, int32_t tokens, int32_t q_heads);
size_t kivi_decode_attn_fp16_workspace(int32_t batch, int32_t kv_heads, int32_t tokens, int32_t q_heads,
                                       int32_t num_splits);

/* Buffer sizes (bytes) for a cache of this shape (pointer fields are ignored):
 * codes = k_codes + v_codes, pairs = k_sz + v_sz, residual = k_res + v_res.  The record
 * kv-efficiency/kivi-2bit-llama2-13b-mha-4k ("KV bytes basis") counts the 2-bit codes as
 * layers x kv heads x head_dim x 2 (K and V) x 2 bits per token and the residual as the
 * newest R tokens in 16-bit floats; codes and residual here are those counts for this cache's
 * capacity (token_cap and residual_cap), and pairs adds the fp16 (scale, zero) per group that
 * the record leaves out (4 bytes per G elements). */
int kivi_cache_bytes(const kivi_cache* shape, size_t* codes, size_t* pairs, size_t* residual);

/* Static description of an error code. */
const char* kivi_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* KIVI_H */
