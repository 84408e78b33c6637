/*
 * kivi_oracle.h -- plain, slow CPU oracle for the KIVI 2-bit KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source, header, table or helper
 * with the HIP library: it re-derives everything (fp16 conversion, the
 * quantizer, the packed layout, attention) from the method's definition.
 *
 * Sources (web pages on KIVI, cited by title and section):
 *  [A] "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *      (summarizepaper export of arXiv 2402.02750v2), title, "Key points", "Summary".
 *  [B] inference-research record kv-efficiency/kivi-2bit-llama2-13b-mha-4k,
 *      fields "Model", "KV bytes basis", "Quant method", "Methodology", "notes".
 *  [C] "Your KV cache doesn't have a bit problem, it has a geometry problem"
 *      (theaiarticle.com), paragraphs 1-4.
 *
 * Readings taken where the pages are silent are listed per function.
 * Every function has a pin in tests/ except where marked "parity unpinned"
 * (none at present).
 */
#ifndef KIVI_ORACLE_H
#define KIVI_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- binary16 <-> binary32, written from the IEEE-754 definitions ---- */
uint16_t kivi_ref_f32_to_f16(float x);        /* round to nearest, ties to even, subnormals kept */
float    kivi_ref_f16_to_f32(uint16_t h);     /* exact widening */
void     kivi_ref_f32_to_f16_array(const float* x, uint16_t* out, size_t n);

/* ---- the 2-bit asymmetric group quantizer ----
 * Quantizes the n values x[0], x[stride], ... (fp16 bit patterns) as one group:
 * zero = min, scale = fp16(fp32((max-min)/3)), code = clamp(rne((x-min)/scale), 0, 3).
 * codes[i] receives the code of x[i*stride] (one code per byte, unpacked). */
void kivi_ref_quant_group(const uint16_t* x, ptrdiff_t stride, int32_t n,
                          uint16_t* scale, uint16_t* zero, uint8_t* codes);
/* The same quantizer with 2^bits levels (bits = 2 or 4): scale = (max - min)/(2^bits - 1),
 * codes clamped to 2^bits - 1. */
void kivi_ref_quant_group_bits(const uint16_t* x, ptrdiff_t stride, int32_t n, int32_t bits,
                               uint16_t* scale, uint16_t* zero, uint8_t* codes);

/* ---- the cache (host memory, same documented layout as the device cache) ----
 * row = b*kv_heads + h.  With bits = 4, k_codes and v_codes are [row][token_cap][head_dim/2]
 * bytes instead (channel j of token t in byte j/2, the even channel in the low nibble).
 *   k_codes, v_codes : [row][token_cap/32][1024] bytes, one 1024-byte tile per 32-token
 *                      group (head_dim 128).
 *                      k_codes: a little-endian 32-bit word holds channels 16w..16w+15 of
 *                      one token, channel 16w+4i+b in byte b at bits 2i, 2i+1; 16-byte chunk
 *                      (16k+n) holds words k, 4+k of token n, then of token 16+n.
 *                      v_codes: a byte holds one channel's codes for four consecutive tokens
 *                      (token 4a+i at bits 2i, 2i+1); 16-byte chunk (16k+n) covers tokens
 *                      8k..8k+7 and channels n+16v, its byte 4p+2h+e holding channel
 *                      n+16(2p+e) for tokens 8k+4h..8k+4h+3.
 *   k_sz             : [row][token_cap/group][head_dim][2] fp16 (scale, zero) per
 *                      (token group, channel)  -- keys per-channel.
 *   v_sz             : [row][token_cap][head_dim/group][2] fp16 (scale, zero) per
 *                      (token, channel group)  -- values per-token.
 *   k_res, v_res     : [row][residual_cap][head_dim] fp16 ring; the n_res residual
 *                      tokens, oldest first, sit in slots (res_head+i) % residual_cap. */
typedef struct kivi_ref_cache {
    int32_t batch, kv_heads, head_dim, group, residual_cap, token_cap;
    int32_t n_quant, n_res, res_head;
    int32_t flush_all;   /* flush policy: 0 = the oldest group of a full residual, 1 = all of it */
    int32_t bits;        /* code width: 2 (default; 0 reads as 2) or 4 */
    uint8_t *k_codes, *v_codes;
    uint16_t *k_sz, *v_sz;
    uint16_t *k_res, *v_res;
} kivi_ref_cache;

/* Keys per-channel: src fp16 [row][tokens][head_dim] with row stride src_row_stride
 * (elements).  Quantizes token groups of `group` tokens into tokens
 * [dst_off, dst_off+tokens) of the cache.  tokens and dst_off are multiples of group. */
void kivi_ref_quantize_k(kivi_ref_cache* c, const uint16_t* src, int32_t tokens,
                         int64_t src_row_stride, int32_t dst_off);
/* Values per-token: every token's channels in groups of `group`. */
void kivi_ref_quantize_v(kivi_ref_cache* c, const uint16_t* src, int32_t tokens,
                         int64_t src_row_stride, int32_t dst_off);

/* Prefill from a context of `tokens` fp16 tokens: the first n_quant (a multiple of
 * group) are quantized, the remaining tokens-n_quant (<= residual_cap) go to ring slots
 * 0.. in order.  Sets n_quant, n_res, res_head=0. */
void kivi_ref_prefill(kivi_ref_cache* c, const uint16_t* k, const uint16_t* v,
                      int32_t tokens, int64_t src_row_stride, int32_t n_quant);

/* One decode-time append of a token per row (k_new, v_new: fp16 [row][head_dim]).
 * If the residual is full, its oldest `group` tokens (flush_all: all residual_cap of
 * them) are first quantized into the next token groups.  Returns 1 if a flush happened,
 * 0 if not. */
int32_t kivi_ref_append(kivi_ref_cache* c, const uint16_t* k_new, const uint16_t* v_new);

/* Materialise the whole context of one row in logical order (quantized history then
 * residual, oldest first) as fp64: K, V are [n_quant+n_res][head_dim]. */
void kivi_ref_dequant_row(const kivi_ref_cache* c, int32_t row, double* K, double* V);

/* Exact-as-fp64 softmax attention of one query q (fp64 [d]) over n keys/values. */
void kivi_ref_attn_dense(const double* q, const double* K, const double* V, int32_t n,
                         int32_t d, double sm_scale, double* out, double* lse);

/* Decode attention of q (fp16 [batch][q_heads][head_dim]) over the cache; query head hq
 * reads kv head hq / (q_heads/kv_heads).  out: fp64 [batch][q_heads][head_dim],
 * lse: fp64 [batch][q_heads] (nullable).  Only rows listed in `rows` (indices
 * b*q_heads+hq) are computed when n_rows > 0; all rows when rows == NULL. */
void kivi_ref_decode_attn(const kivi_ref_cache* c, const uint16_t* q, int32_t q_heads,
                          float sm_scale, double* out, double* lse,
                          const int64_t* rows, int64_t n_rows);

/* Rotary position embedding (rotate-half pairing, w_i = base^(-2i/d)) of x[d] at pos. */
void kivi_ref_rope(const double* x, int32_t d, int64_t pos, double base, double* out);

/* kivi_ref_decode_attn over pre-RoPE keys, each turned at its sequence position. */
void kivi_ref_decode_attn_rope(const kivi_ref_cache* c, const uint16_t* q, int32_t q_heads,
                               float sm_scale, double rope_base, double* out, double* lse,
                               const int64_t* rows, int64_t n_rows);

/* Partial softmax state of one query over keys [t0, t1) of a dense context, and the
 * log-sum-exp merge of such partials.  Used to pin the split-K merge. */
void kivi_ref_attn_partial(const double* q, const double* K, const double* V, int32_t t0,
                           int32_t t1, int32_t d, double sm_scale,
                           double* m, double* l, double* o);
void kivi_ref_attn_merge(const double* m, const double* l, const double* o, int32_t parts,
                         int32_t d, double* out, double* lse);

/* Closed-form byte accounting for a model skeleton (per token, all layers/heads).
 * codes: 2-bit codes for K and V; meta: fp16 (scale, zero) per group for K and V;
 * fp16_token: the same token held in fp16 (one residual token). */
void kivi_ref_bytes_per_token(int64_t layers, int64_t kv_heads, int64_t head_dim,
                              int64_t group, int64_t* codes, int64_t* meta,
                              int64_t* fp16_token);

#ifdef __cplusplus
}
#endif
#endif
