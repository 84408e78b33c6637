/*
 * kivi_oracle.c -- plain, slow CPU oracle for the KIVI 2-bit KV cache.
 *
 * TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's CPU
 * baseline leg use it; the product library never does.  It shares nothing with the
 * HIP library.  Built with gcc -O2 -ffp-contract=off (no fast-math), so every float
 * operation below is one IEEE binary32 operation with a single rounding.
 *
 * Page references (by title and section):
 *  [A] "KIVI: A Tuning-Free Asymmetric 2bit Quantization for KV Cache"
 *      (summarizepaper export of arXiv 2402.02750v2): title, "Key points", "Summary".
 *  [B] inference-research record kv-efficiency/kivi-2bit-llama2-13b-mha-4k:
 *      fields "KV bytes basis", "Quant method", "Methodology".
 *  [C] "Your KV cache doesn't have a bit problem, it has a geometry problem",
 *      paragraphs 1-4.
 *  [D] GrooveSquid summary of "KVQuant: Towards 10 Million Context Length LLM Inference
 *      with KV Cache Quantization": medium-difficulty summary.
 */
#include "kivi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* binary16 <-> binary32 from the IEEE-754 definitions                        */
/* ------------------------------------------------------------------------- */

/* Round a non-negative double to an integer, ties to even. */
static double rne_double(double v) {
    double f = floor(v);
    double frac = v - f;
    if (frac > 0.5) return f + 1.0;
    if (frac < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Subnormals are m * 2^-24, normals (1024+m) * 2^(e-25) for e = 1..30. */
uint16_t kivi_ref_f32_to_f16(float x) {
    uint32_t bits;
    memcpy(&bits, &x, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    double a = fabs((double)x);            /* exact widening */
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    if (isinf(x)) return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {             /* subnormal range: quantum 2^-24 */
        double n = rne_double(a * ldexp(1.0, 24));   /* exact scaling */
        return (uint16_t)(sign | (uint16_t)n);       /* n == 1024 is the smallest normal */
    }
    int e2;
    frexp(a, &e2);                         /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                        /* a in [2^e, 2^(e+1)) */
    double n = rne_double(ldexp(a, 10 - e));   /* significand in units of 2^(e-10) */
    if (n == 2048.0) { n = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7c00u);   /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024.0));
}

float kivi_ref_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = (m == 0) ? INFINITY : NAN;
    else v = ldexp((double)(1024 + m), e - 25);
    return (float)(sign ? -v : v);
}

void kivi_ref_f32_to_f16_array(const float* x, uint16_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = kivi_ref_f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------------- */
/* The asymmetric 2-bit group quantizer                                       */
/* ------------------------------------------------------------------------- */

/* Round a non-negative float to an integer, ties to even. */
static float rne_float(float t) {
    float f = floorf(t);
    float frac = t - f;                    /* exact */
    if (frac > 0.5f) return f + 1.0f;
    if (frac < 0.5f) return f;
    return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
}

/* [A] title and [B] "Methodology": KIVI-2 is an *asymmetric* 2-bit scheme.  Plainest
 * reading: each group keeps its minimum as the zero point and spreads four levels
 * min, min+s, min+2s, min+3s = max over the group's range, s = (max-min)/3.
 * Precision readings: min/max exact; range, s and the per-element quotient in
 * binary32 with one rounding each (true division, no reciprocal); the scale is
 * stored as fp16 (RNE, subnormals kept) and the codes are computed against that
 * stored scale, so a code is the nearest level of the stored (scale, zero);
 * rounding ties go to the even code; a zero scale gives all codes 0; signed zeros
 * are read as +0 for the minimum and maximum, so the zero point and a zero scale are
 * stored as +0 whatever the order of -0 and +0 in the group. */
void kivi_ref_quant_group(const uint16_t* x, ptrdiff_t stride, int32_t n,
                          uint16_t* scale, uint16_t* zero, uint8_t* codes) {
    kivi_ref_quant_group_bits(x, stride, n, 2, scale, zero, codes);
}

/* The same quantizer with 2^bits levels (bits = 2 or 4): s = (max-min)/(2^bits - 1), codes
 * clamped to 2^bits - 1.  KIVI-2 names the 2-bit member of the family; the width is the
 * scheme's parameter. */
void kivi_ref_quant_group_bits(const uint16_t* x, ptrdiff_t stride, int32_t n, int32_t bits,
                               uint16_t* scale, uint16_t* zero, uint8_t* codes) {
    const float top = (float)((1 << bits) - 1);   /* the highest code */
    float mn = INFINITY, mx = -INFINITY;
    for (int32_t i = 0; i < n; ++i) {
        float v = kivi_ref_f16_to_f32(x[i * stride]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    if (mn == 0.0f) mn = 0.0f;             /* canonical +0 zero point */
    if (mx == 0.0f) mx = 0.0f;             /* so a zero range, hence a zero scale, is +0 */
    float range = mx - mn;
    float s32 = range / top;
    uint16_t s16 = kivi_ref_f32_to_f16(s32);
    float s = kivi_ref_f16_to_f32(s16);
    *scale = s16;
    *zero = kivi_ref_f32_to_f16(mn);       /* exact: mn is an fp16 value */
    for (int32_t i = 0; i < n; ++i) {
        if (s == 0.0f) { codes[i] = 0; continue; }
        float v = kivi_ref_f16_to_f32(x[i * stride]);
        float d = v - mn;
        float t = d / s;
        float r = rne_float(t);
        if (r > top) r = top;
        codes[i] = (uint8_t)r;
    }
}

/* ------------------------------------------------------------------------- */
/* Packed layout                                                             */
/* ------------------------------------------------------------------------- */

static int64_t row_count(const kivi_ref_cache* c) { return (int64_t)c->batch * c->kv_heads; }

/* Code positions.  Codes are packed four to a byte, and a row is a sequence of 1024-byte
 * tiles, one per 32-token group.
 *
 * Key tiles: a little-endian 32-bit word holds the 16 channels 16w..16w+15 of one token,
 * channel 16w + 4i + b in byte b at bits 2i, 2i+1.  16-byte chunk (16k + n) (k = 0..3,
 * n = 0..15) holds words k and 4 + k of token n, then words k and 4 + k of token 16 + n.
 *
 * Value tiles: a byte holds one channel's codes for four consecutive tokens, token 4a + i
 * at bits 2i, 2i+1.  16-byte chunk (16k + n) holds, for the 8 tokens 8k..8k+7, the codes
 * of the 8 channels n + 16v (v = 0..7): its byte 4p + 2h + e holds channel n + 16(2p + e)
 * for tokens 8k + 4h .. 8k + 4h + 3 (p = 0..3, h = 0..1, e = 0..1). */
static int64_t key_code_byte(int32_t t, int32_t j) {
    int32_t tt = t % 32, w = j / 16, c = j % 16;
    return (int64_t)(t / 32) * 1024 + ((w % 4) * 16 + tt % 16) * 16 + (tt / 16) * 8 + (w / 4) * 4 + (c % 4);
}
static int key_code_shift(int32_t j) { return 2 * ((j % 16) / 4); }
static int64_t value_code_byte(int32_t t, int32_t j) {
    int32_t tt = t % 32, v = j / 16, n = j % 16;
    return (int64_t)(t / 32) * 1024 + ((tt / 8) * 16 + n) * 16 + (v / 2) * 4 + ((tt % 8) / 4) * 2 + v % 2;
}
static int value_code_shift(int32_t t) { return 2 * (t % 4); }

/* 4-bit codes, keys and values alike: token-major, head_dim/2 bytes per token; channel j
 * of token t in byte j/2, the even channel in the low nibble. */
static int bits_of(const kivi_ref_cache* c) { return c->bits == 4 ? 4 : 2; }

static int64_t code_byte(const kivi_ref_cache* c, int key, int32_t t, int32_t j) {
    if (bits_of(c) == 4) return (int64_t)t * (c->head_dim / 2) + j / 2;
    return key ? key_code_byte(t, j) : value_code_byte(t, j);
}
static int code_shift(const kivi_ref_cache* c, int key, int32_t t, int32_t j) {
    if (bits_of(c) == 4) return 4 * (j % 2);
    return key ? key_code_shift(j) : value_code_shift(t);
}

static void put_code(const kivi_ref_cache* c, uint8_t* codes_row, int key, int32_t t, int32_t j, uint8_t code) {
    uint8_t* byte = codes_row + code_byte(c, key, t, j);
    int sh = code_shift(c, key, t, j);
    unsigned mask = (1u << bits_of(c)) - 1u;
    *byte = (uint8_t)((*byte & ~(mask << sh)) | ((unsigned)code << sh));
}

static uint8_t get_code(const kivi_ref_cache* c, const uint8_t* codes_row, int key, int32_t t, int32_t j) {
    unsigned mask = (1u << bits_of(c)) - 1u;
    return (uint8_t)((codes_row[code_byte(c, key, t, j)] >> code_shift(c, key, t, j)) & mask);
}

static uint8_t* k_codes_row(const kivi_ref_cache* c, int64_t row) {
    return c->k_codes + row * c->token_cap * (c->head_dim * bits_of(c) / 8);
}
static uint8_t* v_codes_row(const kivi_ref_cache* c, int64_t row) {
    return c->v_codes + row * c->token_cap * (c->head_dim * bits_of(c) / 8);
}
/* (scale, zero) of key token group g, channel j */
static uint16_t* k_pair(const kivi_ref_cache* c, int64_t row, int32_t g, int32_t j) {
    int64_t groups = c->token_cap / c->group;
    return c->k_sz + ((row * groups + g) * c->head_dim + j) * 2;
}
/* (scale, zero) of value token t, channel group k */
static uint16_t* v_pair(const kivi_ref_cache* c, int64_t row, int32_t t, int32_t k) {
    int64_t per_tok = c->head_dim / c->group;
    return c->v_sz + ((row * c->token_cap + t) * per_tok + k) * 2;
}
static uint16_t* res_slot(const kivi_ref_cache* c, uint16_t* base, int64_t row, int32_t slot) {
    return base + (row * c->residual_cap + slot) * c->head_dim;
}

/* ------------------------------------------------------------------------- */
/* Keys per-channel, values per-token ([C] paragraphs 1-3; [B] "Quant method")  */
/* ------------------------------------------------------------------------- */

/* Keys: for each channel j, the `group` consecutive tokens of a token group form one
 * quantization group (per-channel quantization isolates the fixed outlier channels). */
void kivi_ref_quantize_k(kivi_ref_cache* c, const uint16_t* src, int32_t tokens,
                         int64_t src_row_stride, int32_t dst_off) {
    int32_t d = c->head_dim, G = c->group;
    uint8_t* codes = (uint8_t*)malloc((size_t)G);
    for (int64_t row = 0; row < row_count(c); ++row) {
        const uint16_t* s_row = src + row * src_row_stride;
        for (int32_t g = 0; g < tokens / G; ++g) {
            int32_t t0 = g * G;                       /* first source token */
            int32_t cg = (dst_off + t0) / G;          /* destination token group */
            for (int32_t j = 0; j < d; ++j) {
                uint16_t* pr = k_pair(c, row, cg, j);
                kivi_ref_quant_group_bits(s_row + (int64_t)t0 * d + j, d, G, bits_of(c), &pr[0], &pr[1], codes);
                for (int32_t i = 0; i < G; ++i)
                    put_code(c, k_codes_row(c, row), 1, dst_off + t0 + i, j, codes[i]);
            }
        }
    }
    free(codes);
}

/* Values: for each token, each run of `group` consecutive channels is one group. */
void kivi_ref_quantize_v(kivi_ref_cache* c, const uint16_t* src, int32_t tokens,
                         int64_t src_row_stride, int32_t dst_off) {
    int32_t d = c->head_dim, G = c->group;
    uint8_t* codes = (uint8_t*)malloc((size_t)G);
    for (int64_t row = 0; row < row_count(c); ++row) {
        const uint16_t* s_row = src + row * src_row_stride;
        for (int32_t t = 0; t < tokens; ++t) {
            for (int32_t k = 0; k < d / G; ++k) {
                uint16_t* pr = v_pair(c, row, dst_off + t, k);
                kivi_ref_quant_group_bits(s_row + (int64_t)t * d + k * G, 1, G, bits_of(c), &pr[0], &pr[1], codes);
                for (int32_t i = 0; i < G; ++i)
                    put_code(c, v_codes_row(c, row), 0, dst_off + t, k * G + i, codes[i]);
            }
        }
    }
    free(codes);
}

/* ------------------------------------------------------------------------- */
/* Residual and group flush ([C] paragraph 4; [B] "KV bytes basis")           */
/* ------------------------------------------------------------------------- */

void kivi_ref_prefill(kivi_ref_cache* c, const uint16_t* k, const uint16_t* v,
                      int32_t tokens, int64_t src_row_stride, int32_t n_quant) {
    int32_t d = c->head_dim;
    kivi_ref_quantize_k(c, k, n_quant, src_row_stride, 0);
    kivi_ref_quantize_v(c, v, n_quant, src_row_stride, 0);
    for (int64_t row = 0; row < row_count(c); ++row)
        for (int32_t i = 0; i < tokens - n_quant; ++i) {
            memcpy(res_slot(c, c->k_res, row, i), k + row * src_row_stride + (int64_t)(n_quant + i) * d, (size_t)d * 2);
            memcpy(res_slot(c, c->v_res, row, i), v + row * src_row_stride + (int64_t)(n_quant + i) * d, (size_t)d * 2);
        }
    c->n_quant = n_quant;
    c->n_res = tokens - n_quant;
    c->res_head = 0;
}

/* The record's byte basis keeps the most recent R tokens in full precision and
 * quantizes only whole token groups of history.  Reading of the flush policy: when a
 * token arrives and the residual already holds R tokens, the oldest `group` of them
 * become the next quantized token group (keys and values together), then the new
 * token enters the residual.  The other policy (flush_all; the summary page's ablation
 * over the residual length, where the residual is the full-precision buffer that fills
 * up): all R residual tokens become the next R/group token groups. */
int32_t kivi_ref_append(kivi_ref_cache* c, const uint16_t* k_new, const uint16_t* v_new) {
    int32_t d = c->head_dim, R = c->residual_cap;
    int32_t G = c->flush_all ? R : c->group;   /* tokens flushed: whole groups either way */
    int32_t flushed = 0;
    if (c->n_res == R) {
        uint16_t* kt = (uint16_t*)malloc((size_t)G * d * 2);
        uint16_t* vt = (uint16_t*)malloc((size_t)G * d * 2);
        for (int64_t row = 0; row < row_count(c); ++row) {
            for (int32_t i = 0; i < G; ++i) {   /* oldest G residual tokens, in order */
                int32_t slot = (c->res_head + i) % R;
                memcpy(kt + (int64_t)i * d, res_slot(c, c->k_res, row, slot), (size_t)d * 2);
                memcpy(vt + (int64_t)i * d, res_slot(c, c->v_res, row, slot), (size_t)d * 2);
            }
            /* quantize this one row's tile: reuse the per-row loops on a 1-row view */
            kivi_ref_cache one = *c;
            one.batch = 1;
            one.kv_heads = 1;
            one.k_codes = k_codes_row(c, row);
            one.v_codes = v_codes_row(c, row);
            one.k_sz = k_pair(c, row, 0, 0);
            one.v_sz = v_pair(c, row, 0, 0);
            kivi_ref_quantize_k(&one, kt, G, (int64_t)G * d, c->n_quant);
            kivi_ref_quantize_v(&one, vt, G, (int64_t)G * d, c->n_quant);
        }
        free(kt);
        free(vt);
        c->n_quant += G;
        c->res_head = (c->res_head + G) % R;
        c->n_res -= G;
        flushed = 1;
    }
    int32_t slot = (c->res_head + c->n_res) % R;
    for (int64_t row = 0; row < row_count(c); ++row) {
        memcpy(res_slot(c, c->k_res, row, slot), k_new + row * d, (size_t)d * 2);
        memcpy(res_slot(c, c->v_res, row, slot), v_new + row * d, (size_t)d * 2);
    }
    c->n_res += 1;
    return flushed;
}

/* ------------------------------------------------------------------------- */
/* Dequantization and attention                                              */
/* ------------------------------------------------------------------------- */

/* x_hat = zero + code * scale, exact in fp64. */
void kivi_ref_dequant_row(const kivi_ref_cache* c, int32_t row, double* K, double* V) {
    int32_t d = c->head_dim, G = c->group;
    for (int32_t t = 0; t < c->n_quant; ++t) {
        for (int32_t j = 0; j < d; ++j) {
            const uint16_t* kp = k_pair(c, row, t / G, j);
            const uint16_t* vp = v_pair(c, row, t, j / G);
            double kc = get_code(c, k_codes_row(c, row), 1, t, j);
            double vc = get_code(c, v_codes_row(c, row), 0, t, j);
            K[(int64_t)t * d + j] = (double)kivi_ref_f16_to_f32(kp[1]) + kc * (double)kivi_ref_f16_to_f32(kp[0]);
            V[(int64_t)t * d + j] = (double)kivi_ref_f16_to_f32(vp[1]) + vc * (double)kivi_ref_f16_to_f32(vp[0]);
        }
    }
    for (int32_t i = 0; i < c->n_res; ++i) {
        int32_t slot = (c->res_head + i) % c->residual_cap;
        const uint16_t* kr = res_slot(c, c->k_res, row, slot);
        const uint16_t* vr = res_slot(c, c->v_res, row, slot);
        for (int32_t j = 0; j < d; ++j) {
            K[(int64_t)(c->n_quant + i) * d + j] = kivi_ref_f16_to_f32(kr[j]);
            V[(int64_t)(c->n_quant + i) * d + j] = kivi_ref_f16_to_f32(vr[j]);
        }
    }
}

/* softmax(sm_scale * q.K^T) . V in fp64; lse = log of the softmax denominator. */
void kivi_ref_attn_dense(const double* q, const double* K, const double* V, int32_t n,
                         int32_t d, double sm_scale, double* out, double* lse) {
    double* logit = (double*)malloc((size_t)n * sizeof(double));
    double m = -INFINITY;
    for (int32_t t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int32_t j = 0; j < d; ++j) acc += q[j] * K[(int64_t)t * d + j];
        logit[t] = sm_scale * acc;
        if (logit[t] > m) m = logit[t];
    }
    double l = 0.0;
    for (int32_t j = 0; j < d; ++j) out[j] = 0.0;
    for (int32_t t = 0; t < n; ++t) {
        double p = exp(logit[t] - m);
        l += p;
        for (int32_t j = 0; j < d; ++j) out[j] += p * V[(int64_t)t * d + j];
    }
    for (int32_t j = 0; j < d; ++j) out[j] /= l;
    if (lse) *lse = m + log(l);
    free(logit);
}

void kivi_ref_decode_attn(const kivi_ref_cache* c, const uint16_t* q, int32_t q_heads,
                          float sm_scale, double* out, double* lse,
                          const int64_t* rows, int64_t n_rows) {
    int32_t d = c->head_dim;
    int32_t n = c->n_quant + c->n_res;
    int32_t ratio = q_heads / c->kv_heads;       /* query heads per kv head */
    int64_t total = (int64_t)c->batch * q_heads;
    double* K = (double*)malloc((size_t)n * d * sizeof(double));
    double* V = (double*)malloc((size_t)n * d * sizeof(double));
    double* qd = (double*)malloc((size_t)d * sizeof(double));
    int64_t last_kv_row = -1;
    int64_t count = rows ? n_rows : total;
    for (int64_t idx = 0; idx < count; ++idx) {
        int64_t r = rows ? rows[idx] : idx;      /* r = b*q_heads + hq */
        int64_t b = r / q_heads, hq = r % q_heads;
        int64_t kv_row = b * c->kv_heads + hq / ratio;
        if (kv_row != last_kv_row) {
            kivi_ref_dequant_row(c, (int32_t)kv_row, K, V);
            last_kv_row = kv_row;
        }
        for (int32_t j = 0; j < d; ++j) qd[j] = kivi_ref_f16_to_f32(q[r * d + j]);
        kivi_ref_attn_dense(qd, K, V, n, d, (double)sm_scale, out + r * d, lse ? lse + r : NULL);
    }
    free(K);
    free(V);
    free(qd);
}

/* Rotary position embedding of one vector at position pos.  [C] paragraph 4 and [D] advise
 * quantizing keys before RoPE is applied, so the rotation comes after dequantization; the
 * pages name RoPE without writing it out.  Reading: the rotary embedding with the
 * rotate-half pairing of the Llama-2 models the pages measure -- channel i < d/2 pairs
 * with channel i + d/2, pair i turns at frequency w_i = base^(-2i/d), and a token at
 * position pos is turned by the angle pos*w_i:
 *   out_i = x_i cos - x_{i+d/2} sin,   out_{i+d/2} = x_{i+d/2} cos + x_i sin.
 * All in binary64 with the C library's pow, cos and sin. */
void kivi_ref_rope(const double* x, int32_t d, int64_t pos, double base, double* out) {
    int32_t h = d / 2;
    for (int32_t i = 0; i < h; ++i) {
        double w = pow(base, -2.0 * (double)i / (double)d);
        double a = (double)pos * w;
        double cs = cos(a), sn = sin(a);
        double x0 = x[i], x1 = x[i + h];
        out[i] = x0 * cs - x1 * sn;
        out[i + h] = x1 * cs + x0 * sn;
    }
}

/* Decode attention over a cache of pre-RoPE keys: every key is dequantized (history) or
 * read (fp16 residual), then turned by kivi_ref_rope at its position in the sequence --
 * history token t at position t, the i-th oldest residual token at n_quant + i -- and
 * the query (already rotated by the caller at its own position) attends over the turned
 * keys as in kivi_ref_decode_attn.  Values carry no position and are used as they are. */
void kivi_ref_decode_attn_rope(const kivi_ref_cache* c, const uint16_t* q, int32_t q_heads,
                               float sm_scale, double rope_base, double* out, double* lse,
                               const int64_t* rows, int64_t n_rows) {
    int32_t d = c->head_dim;
    int32_t n = c->n_quant + c->n_res;
    int32_t ratio = q_heads / c->kv_heads;
    int64_t total = (int64_t)c->batch * q_heads;
    double* K = (double*)malloc((size_t)n * d * sizeof(double));
    double* Kr = (double*)malloc((size_t)n * d * sizeof(double));
    double* V = (double*)malloc((size_t)n * d * sizeof(double));
    double* qd = (double*)malloc((size_t)d * sizeof(double));
    int64_t last_kv_row = -1;
    int64_t count = rows ? n_rows : total;
    for (int64_t idx = 0; idx < count; ++idx) {
        int64_t r = rows ? rows[idx] : idx;
        int64_t b = r / q_heads, hq = r % q_heads;
        int64_t kv_row = b * c->kv_heads + hq / ratio;
        if (kv_row != last_kv_row) {
            kivi_ref_dequant_row(c, (int32_t)kv_row, K, V);
            for (int32_t t = 0; t < n; ++t) kivi_ref_rope(K + (int64_t)t * d, d, t, rope_base, Kr + (int64_t)t * d);
            last_kv_row = kv_row;
        }
        for (int32_t j = 0; j < d; ++j) qd[j] = kivi_ref_f16_to_f32(q[r * d + j]);
        kivi_ref_attn_dense(qd, Kr, V, n, d, (double)sm_scale, out + r * d, lse ? lse + r : NULL);
    }
    free(K);
    free(Kr);
    free(V);
    free(qd);
}

/* Softmax state over keys [t0, t1): m = max logit, l = sum exp(logit - m),
 * o = sum exp(logit - m) * v (unnormalised). */
void kivi_ref_attn_partial(const double* q, const double* K, const double* V, int32_t t0,
                           int32_t t1, int32_t d, double sm_scale,
                           double* m, double* l, double* o) {
    double mm = -INFINITY;
    for (int32_t t = t0; t < t1; ++t) {
        double acc = 0.0;
        for (int32_t j = 0; j < d; ++j) acc += q[j] * K[(int64_t)t * d + j];
        if (sm_scale * acc > mm) mm = sm_scale * acc;
    }
    double ll = 0.0;
    for (int32_t j = 0; j < d; ++j) o[j] = 0.0;
    for (int32_t t = t0; t < t1; ++t) {
        double acc = 0.0;
        for (int32_t j = 0; j < d; ++j) acc += q[j] * K[(int64_t)t * d + j];
        double p = exp(sm_scale * acc - mm);
        ll += p;
        for (int32_t j = 0; j < d; ++j) o[j] += p * V[(int64_t)t * d + j];
    }
    *m = mm;
    *l = ll;
}

/* Merge: m* = max m_s, l* = sum l_s e^(m_s - m*), out = sum o_s e^(m_s - m*) / l*,
 * lse = m* + log l*.  Empty parts carry m = -inf, l = 0 and are skipped. */
void kivi_ref_attn_merge(const double* m, const double* l, const double* o, int32_t parts,
                         int32_t d, double* out, double* lse) {
    double ms = -INFINITY;
    for (int32_t s = 0; s < parts; ++s)
        if (m[s] > ms) ms = m[s];
    double ls = 0.0;
    for (int32_t j = 0; j < d; ++j) out[j] = 0.0;
    for (int32_t s = 0; s < parts; ++s) {
        if (l[s] == 0.0) continue;
        double w = exp(m[s] - ms);
        ls += l[s] * w;
        for (int32_t j = 0; j < d; ++j) out[j] += o[(int64_t)s * d + j] * w;
    }
    for (int32_t j = 0; j < d; ++j) out[j] /= ls;
    if (lse) *lse = ms + log(ls);
}

/* ------------------------------------------------------------------------- */
/* Byte accounting ([B] "KV bytes basis")                                    */
/* ------------------------------------------------------------------------- */

/* Per token over all layers and kv heads: codes = layers*heads*d*2(K,V)*2 bits/8;
 * meta = one fp16 (scale, zero) pair per `group` elements of K and of V;
 * fp16_token = layers*heads*d*2(K,V)*2 bytes. */
void kivi_ref_bytes_per_token(int64_t layers, int64_t kv_heads, int64_t head_dim,
                              int64_t group, int64_t* codes, int64_t* meta,
                              int64_t* fp16_token) {
    int64_t elems = layers * kv_heads * head_dim * 2;   /* K and V elements per token */
    *codes = elems * 2 / 8;
    *meta = (elems / group) * 2 * 2;                    /* (scale, zero), 2 bytes each */
    *fp16_token = elems * 2;
}
