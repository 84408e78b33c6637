// kivi_quant.hip -- quantize, prefill, append and group-flush kernels (gfx950).
//
// Keys are quantized per-channel over groups of G tokens, values per-token over groups
// of G channels, G = 32 by default and 64 or 128 as the pages' ablation parameter (record
// kv-efficiency/kivi-2bit-llama2-13b-mha-4k, "Quant method"; article "Your KV cache
// doesn't have a bit problem...", paragraphs 2-3; KIVI summary, "Key points": group size
// G and residual length R as hyperparameters).  Codes are stored in 32-token tiles
// whatever G is.
// The newest R tokens stay in fp16 and whole groups of the oldest residual tokens are
// moved into the quantized history (record, "KV bytes basis").
//
// All kernels use 256-thread workgroups and 16-byte global accesses.
#include <algorithm>

#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

constexpr int kQSlots = kD + kD / 16;   // key-group threshold slots in LDS (quant_k_group)

// 2-bit codes without a division.  The code of x is min(rint(fl(d / s)), 3) with d = fl(x - mn),
// fl the binary32 rounding and rint ties-to-even, so it steps only where fl(d / s) crosses 0.5,
// 1.5 and 2.5.  With round-to-nearest-even those crossings sit at fixed points of the exact
// quotient: code >= 1 iff d/s > 0.5 + 2^-25 (the midpoint above 0.5, whose tie goes to 0.5),
// code >= 2 iff d/s >= 1.5 - 2^-24 (the midpoint below 1.5, whose tie goes to 1.5), code >= 3
// iff d/s > 2.5 + 2^-23.  For s > 0 each is a comparison of d with m*s, exact in binary64 (s
// has 11 significant bits, m at most 25), and for a binary32 d, d > T iff d > RD(T) and
// d >= T iff d >= RU(T) (RD, RU: the binary32 neighbours of T below and above).  So three
// thresholds per group give every code of the group with three comparisons, for every finite
// input (s = 0, a constant group, gives code 0).
struct GroupT {
    float mn, t1, t2, t3;
    uint32_t pair;
};
__device__ __forceinline__ float f32_down(double x) {   // the largest binary32 <= x (x >= 0)
    const float f = (float)x;
    return (double)f > x ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) - 1u) : f;
}
__device__ __forceinline__ float f32_up(double x) {     // the smallest binary32 >= x (x >= 0)
    const float f = (float)x;
    return (double)f < x ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) + 1u) : f;
}
__device__ __forceinline__ GroupT group_thresholds(float mn, float mx) {
    const GroupQ q = group_params(mn, mx);
    GroupT g;
    g.mn = q.mn;
    g.pair = q.pair;
    if (q.s == 0.0f) {
        g.t1 = g.t2 = g.t3 = __builtin_inff();
    } else {
        const double s = (double)q.s;
        g.t1 = f32_down(s * (0.5 + 0x1p-25));
        g.t2 = f32_up(s * (1.5 - 0x1p-24));
        g.t3 = f32_down(s * (2.5 + 0x1p-23));
    }
    return g;
}
__device__ __forceinline__ uint32_t code2_of(float x, float mn, float t1, float t2, float t3) {
#pragma clang fp contract(off)
    const float d = x - mn;
    return (uint32_t)(d > t1) + (uint32_t)(d >= t2) + (uint32_t)(d > t3);
}

// The same rule on the fp16 inputs themselves, two at a time.  The thresholds are the exact
// binary32 products t1 = s/2, t2 = 3s/2, t3 = 5s/2 (s has 11 significant bits, so the binary32
// neighbours of (0.5 + 2^-25)s, (1.5 - 2^-24)s and (2.5 + 2^-23)s are these products
// themselves), and each step is [fl(x - mn) > s/2], [fl(x - mn) > u2]
// (u2 the binary32 below 3s/2) or [fl(x - mn) > 5s/2]: monotone in x, so it holds exactly for
// the fp16 x above one fp16 bound V.  fl(y) <= u iff y <= u + ulp(u)/2 when u is even (s/2
// and 5s/2 are: the midpoint's tie rounds to them) and y < u + ulp(u)/2 when u is odd (u2:
// u2 + ulp/2 = 3s/2 - ulp(3s/2)/2, 3s/2 never a power of two).  So V is the largest fp16 at or
// below mn + s/2 + ulp(s/2)/2, below mn + 3s/2 - ulp(3s/2)/2, at or below mn + 5s/2 +
// ulp(5s/2)/2.  Those sums are formed in binary64, where they are exact (mn has 11 significant
// bits and the other terms 25 at most, within a span binary64 holds for any group whose range
// is not 0), rounded to fp16 through binary32 (RNE twice: at most one step too high) and moved
// one step down where that overshoots.  A constant group (s = 0) gets V = inf.  Then x > V is
// the sign of the fp16 difference V - x: rounding keeps the sign of a nonzero difference
// (overflow to inf and underflow to -0 included), equal values give +0, and V is never -0.
// So a pair of codes is three packed fp16 subtractions, three packed shifts and one add.  A
// restatement of these bounds gives the division's code for every finite fp16 minimum and
// every positive fp16 scale (tests/test_code_bounds.py checks a spread of them on the CPU).
__device__ __forceinline__ uint32_t prev_f16(uint32_t h) {   // the fp16 below h (h not -inf)
    return (h & 0x7fffu) == 0 ? 0x8001u : ((h & 0x8000u) ? h + 1u : h - 1u);
}
template <bool STRICT>   // the largest fp16 at or below S (STRICT: below S)
__device__ __forceinline__ uint32_t f16_floor(double S) {
    float f = (float)S;
    asm volatile("" : "+v"(f));   // two hardware conversions, not one emulated binary64 -> fp16
    const uint32_t h = f2h(f);
    const double hd = (double)h2f(h);
    return (STRICT ? hd >= S : hd > S) ? prev_f16(h) : h;
}
__device__ __forceinline__ double half_ulp(float v) {   // ulp(v)/2 of a normal positive binary32
    return __builtin_ldexp(1.0, __builtin_amdgcn_frexp_expf(v) - 25);
}
struct GroupV {
    uint32_t pair;         // (scale, zero) word
    uint32_t v1, v2, v3;   // fp16 bounds of the three code steps
};
__device__ __forceinline__ GroupV group_bounds(float mn, float mx) {
    const GroupQ q = group_params(mn, mx);
    GroupV b;
    b.pair = q.pair;
    if (q.s == 0.0f) {
        b.v1 = b.v2 = b.v3 = 0x7c00u;
    } else {
        const double m = (double)q.mn;
        const float s1 = 0.5f * q.s, s2 = 1.5f * q.s, s3 = 2.5f * q.s;   // exact
        b.v1 = f16_floor<false>(m + ((double)s1 + half_ulp(s1)));
        b.v2 = f16_floor<true>(m + ((double)s2 - half_ulp(s2)));
        b.v3 = f16_floor<false>(m + ((double)s3 + half_ulp(s3)));
    }
    return b;
}
typedef _Float16 hv2 __attribute__((ext_vector_type(2)));
typedef uint16_t uv2 __attribute__((ext_vector_type(2)));
// codes (bits 0..1 and 16..17) of the two fp16 values of x; v1..v3: a bound in both halves
__device__ __forceinline__ uint32_t code_pair(uint32_t x, uint32_t v1, uint32_t v2, uint32_t v3) {
    const hv2 xv = __builtin_bit_cast(hv2, x);
    const uv2 s1 = __builtin_bit_cast(uv2, __builtin_bit_cast(hv2, v1) - xv) >> 15;
    const uv2 s2 = __builtin_bit_cast(uv2, __builtin_bit_cast(hv2, v2) - xv) >> 15;
    const uv2 s3 = __builtin_bit_cast(uv2, __builtin_bit_cast(hv2, v3) - xv) >> 15;
    return __builtin_bit_cast(uint32_t, s1) + __builtin_bit_cast(uint32_t, s2) + __builtin_bit_cast(uint32_t, s3);
}
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_minimum(__builtin_bit_cast(hv2, a), __builtin_bit_cast(hv2, b)));
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_bit_cast(hv2, a), __builtin_bit_cast(hv2, b)));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {   // quad_perm / row rotation, every lane sourced
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int PATTERN>
__device__ __forceinline__ uint32_t swz_u(uint32_t v) {   // ds_swizzle, bit-mask mode (32-lane groups)
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, PATTERN);
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kRowRor8 = 0x128;
constexpr int kSwzXor4 = 0x101F;

// One key token group of GS tokens held in LDS as fp16 [GS][128] -> its GS/32 code tiles +
// 128 pairs.  Called by all 256 threads of the workgroup; ends with the codes and pairs
// stored.  sh_q: LDS [kQSlots], each channel's minimum and code thresholds (group_thresholds),
// channel j at j + j/16 (the 16-channel blocks one slot apart: the eight blocks a wave reads at
// once then sit in different banks).
template <int GS>
__device__ void quant_k_group(const uint16_t* __restrict__ tile, float4* sh_q,
                              uint8_t* __restrict__ codes_dst,      // the group's first code tile
                              uint32_t* __restrict__ pairs_dst) {   // 128 (scale, zero) words
    const int tid = threadIdx.x;
    if (tid < kD) {
        float mn = h2f(tile[tid]), mx = mn;
#pragma unroll 8
        for (int t = 1; t < GS; ++t) {
            float v = h2f(tile[t * kD + tid]);
            mn = __builtin_fminf(mn, v);
            mx = __builtin_fmaxf(mx, v);
        }
        const GroupT g = group_thresholds(mn, mx);
        pairs_dst[tid] = g.pair;
        sh_q[tid + (tid >> 4)] = make_float4(g.mn, g.t1, g.t2, g.t3);
    }
    __syncthreads();
    // thread -> (token t, 16-channel word w) of each 32-token tile: 32 tokens x 8 words
    const int t = tid >> 3, w = tid & 7;
#pragma unroll
    for (int tl = 0; tl < GS / kG; ++tl) {
        const uint4* src = reinterpret_cast<const uint4*>(tile + (tl * kG + t) * kD + w * 16);
        uint4 a = src[0], b = src[1];
        uint32_t h[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t word = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            uint32_t bits = (c & 1) ? (h[c >> 1] >> 16) : (h[c >> 1] & 0xffffu);
            const float4 g = sh_q[w * 17 + c];
            word |= code2_of(h2f(bits), g.x, g.y, g.z, g.w) << code_bit(c);
        }
        *reinterpret_cast<uint32_t*>(codes_dst + tl * kTileBytes + key_word_offset(t, w)) = word;
    }
}

// One 32-token value tile by the whole workgroup.  Tokens lo..hi-1 (tile-local) are
// quantized from src_lo (token t at src_lo + (t - lo)*src_tok_stride, 128 fp16 channels);
// their codes and (scale, zero) words are stored and the codes of the tile's other tokens
// are kept.
// sh_codes: LDS scratch [32][128] bytes.  All 256 threads must call it.  Groups of GS
// channels: the GS/16 lanes of a group reduce its min and max.
template <int GS>
__device__ void quant_v_tile(const uint16_t* __restrict__ src_lo, int64_t src_tok_stride, int lo, int hi,
                             uint8_t (*sh_codes)[kD], uint8_t* __restrict__ tile_dst,
                             uint32_t* __restrict__ pairs_dst) {   // pair word of tile token 0, group 0
    const int tid = threadIdx.x;
    // thread -> (token t, 16-channel block cb); the blocks of a channel group are adjacent
    // lanes
    const int t = tid >> 3, cb = tid & 7;
    const bool live = t >= lo && t < hi;
    uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
    if (live) {
        const uint4* p = reinterpret_cast<const uint4*>(src_lo + (t - lo) * src_tok_stride + cb * 16);
        x0 = p[0];
        x1 = p[1];
    }
    const uint32_t h[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float v[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = h2f(h[i] & 0xffffu);
        v[2 * i + 1] = h2f(h[i] >> 16);
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        mn = __builtin_fminf(mn, v[i]);
        mx = __builtin_fmaxf(mx, v[i]);
    }
#pragma unroll
    for (int m = 1; m < GS / 16; m <<= 1) {
        mn = __builtin_fminf(mn, __shfl_xor(mn, m, 64));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, 64));
    }
    const GroupT q = group_thresholds(mn, mx);
    uint32_t packed[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        packed[w] = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) packed[w] |= code2_of(v[4 * w + b], q.mn, q.t1, q.t2, q.t3) << (8 * b);
    }
    *reinterpret_cast<uint4*>(&sh_codes[t][cb * 16]) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if (live && cb % (GS / 16) == 0) pairs_dst[value_pair_index<GS>(t, cb / (GS / 16))] = q.pair;
    __syncthreads();
    // thread -> 32-bit word tid of the tile: chunk L = tid/4 (tokens 8kg.., channel n + 16v),
    // word p = tid%4; its byte 2hh + e holds channel n + 32p + 16e for tokens 8kg + 4hh + i
    const int L = tid >> 2, p = tid & 3, kg = L >> 4, n = L & 15;
    uint32_t word = 0, mask = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int ch = n + 32 * p + 16 * (b & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = 8 * kg + 4 * (b >> 1) + i;
            if (tt >= lo && tt < hi) {
                word |= (uint32_t)sh_codes[tt][ch] << (8 * b + 2 * i);
                mask |= 3u << (8 * b + 2 * i);
            }
        }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile_dst) + tid;
    if (mask == 0xffffffffu) *dst = word;
    else if (mask != 0u) *dst = (*dst & ~mask) | word;
    __syncthreads();   // sh_codes may be reused by the caller
}

// ---- 4-bit codes (the scheme's 4-bit member: sixteen levels).  Token-major: a token's 128
// codes in 64 bytes, channel j in byte j/2, the even channel in the low nibble.

// One key token group of GS tokens held in LDS as fp16 [GS][128] -> its GS token rows of
// codes (from codes_dst, 64 bytes each) + 128 pairs.  All 256 threads.
template <int GS>
__device__ void quant_k4_group(const uint16_t* __restrict__ tile, float* sh_mn, float* sh_s,
                               uint8_t* __restrict__ codes_dst, uint32_t* __restrict__ pairs_dst) {
    const int tid = threadIdx.x;
    if (tid < kD) {
        float mn = h2f(tile[tid]), mx = mn;
#pragma unroll 8
        for (int t = 1; t < GS; ++t) {
            const float v = h2f(tile[t * kD + tid]);
            mn = __builtin_fminf(mn, v);
            mx = __builtin_fmaxf(mx, v);
        }
        const GroupQ q = group_params<15>(mn, mx);
        pairs_dst[tid] = q.pair;
        sh_mn[tid] = q.mn;
        sh_s[tid] = q.s;
    }
    __syncthreads();
    // item -> (token t, 16-channel chunk w): 8 bytes of codes, channel 16w + c at bit 4c
    for (int i = tid; i < GS * 8; i += kBlock) {
        const int t = i >> 3, w = i & 7;
        const uint4* src = reinterpret_cast<const uint4*>(tile + t * kD + w * 16);
        const uint4 a = src[0], b = src[1];
        const uint32_t h[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int j = w * 16 + c;
            const GroupQ q{sh_mn[j], sh_s[j], 0u};
            const uint32_t code = code_of<15>(h2f((c & 1) ? (h[c >> 1] >> 16) : (h[c >> 1] & 0xffffu)), q);
            if (c < 8) lo |= code << (4 * c);
            else hi |= code << (4 * (c - 8));
        }
        *reinterpret_cast<uint2*>(codes_dst + (int64_t)t * kRowBytes4 + w * 8) = make_uint2(lo, hi);
    }
    __syncthreads();   // the LDS tile and sh_mn / sh_s may be reused by the caller
}

// Value tokens [0, n) from src (token t at src + t*src_tok_stride, 128 fp16 channels) ->
// 4-bit codes (token rows of 64 bytes from codes_dst) and (scale, zero) words (pairs_dst:
// the word of token 0, group 0).  All 256 threads: four per token (32 channels each), 64
// tokens a pass; a group of GS channels is reduced over its GS/32 adjacent lanes.
template <int GS>
__device__ void quant_v4_tokens(const uint16_t* __restrict__ src, int64_t src_tok_stride, int n,
                                uint8_t* __restrict__ codes_dst, uint32_t* __restrict__ pairs_dst) {
    const int tid = threadIdx.x, qd = tid & 3;
    for (int base = 0; base < n; base += kBlock / 4) {
        const int t = base + (tid >> 2);
        const bool live = t < n;
        float v[32];
        const uint4* p = reinterpret_cast<const uint4*>(src + (int64_t)(live ? t : 0) * src_tok_stride + qd * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 x = p[i];
            const uint32_t h[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[8 * i + 2 * k] = h2f(h[k] & 0xffffu);
                v[8 * i + 2 * k + 1] = h2f(h[k] >> 16);
            }
        }
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) {
            mn = __builtin_fminf(mn, v[i]);
            mx = __builtin_fmaxf(mx, v[i]);
        }
#pragma unroll
        for (int m = 1; m < GS / 32; m <<= 1) {
            mn = __builtin_fminf(mn, __shfl_xor(mn, m, 64));
            mx = __builtin_fmaxf(mx, __shfl_xor(mx, m, 64));
        }
        const GroupQ q = group_params<15>(mn, mx);
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = 0;
#pragma unroll
            for (int c = 0; c < 8; ++c) w[i] |= code_of<15>(v[8 * i + c], q) << (4 * c);
        }
        if (live) {
            *reinterpret_cast<uint4*>(codes_dst + (int64_t)t * kRowBytes4 + qd * 16) = make_uint4(w[0], w[1], w[2], w[3]);
            if (qd % (GS / 32) == 0) pairs_dst[value_pair_index<GS>(t, qd / (GS / 32))] = q.pair;
        }
    }
}

// ------------------------------------------------------------------ kernels ------

// grid.x = rows * (tokens / GS); one key token group per workgroup.
template <int GS>
__global__ __launch_bounds__(kBlock) void quantize_k_kernel(QuantArgs a) {
    __shared__ uint4 tile4[GS * kD / 8];
    __shared__ float4 sh_q[kQSlots];
    const int groups = a.tokens / GS;
    const int64_t row = blockIdx.x / groups;
    const int g = blockIdx.x % groups;
    const uint16_t* src = a.src + row * a.src_row_stride + (int64_t)g * GS * kD;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int i = threadIdx.x; i < GS * kD / 8; i += kBlock) tile4[i] = s4[i];
    __syncthreads();
    const int dst_tok = a.dst_token_off + g * GS;
    uint8_t* codes = a.k_codes + row * a.token_cap * kRowBytes + (int64_t)(dst_tok / kG) * kTileBytes;
    uint32_t* pairs = reinterpret_cast<uint32_t*>(a.k_sz) + (row * (a.token_cap / GS) + dst_tok / GS) * kD;
    quant_k_group<GS>(reinterpret_cast<const uint16_t*>(tile4), sh_q, codes, pairs);
}

// grid.x = rows * (32-token tiles touched by [dst_token_off, dst_token_off + tokens)).
template <int GS>
__global__ __launch_bounds__(kBlock) void quantize_v_kernel(QuantArgs a) {
    __shared__ __align__(16) uint8_t sh_codes[kG][kD];
    const int first = a.dst_token_off / kG;
    const int n_tiles = (a.dst_token_off + a.tokens - 1) / kG - first + 1;
    const int64_t row = blockIdx.x / n_tiles;
    const int tile = first + (int)(blockIdx.x % n_tiles);
    const int t0 = tile * kG;                                   // first token of the tile
    const int lo = max(a.dst_token_off, t0) - t0;
    const int hi = min(a.dst_token_off + a.tokens, t0 + kG) - t0;
    // source token of tile token lo: t0 + lo - dst_token_off
    const uint16_t* src = a.src + row * a.src_row_stride + (int64_t)(t0 + lo - a.dst_token_off) * kD;
    quant_v_tile<GS>(src, kD, lo, hi, sh_codes, a.v_codes + (row * a.token_cap + t0) * kRowBytes,
                     reinterpret_cast<uint32_t*>(a.v_sz) + value_pair_index<GS>(row * a.token_cap + t0, 0));
}

// ---- 2-bit quantizers at G = 32 for whole ranges of tokens (prefill).  One wave per work
// item, no LDS tile and no workgroup barrier: a lane loads 16 bytes (8 channels) of each of
// four tokens and keeps them in registers; the group minima and maxima are packed fp16 minima
// and maxima, reduced across lanes with DPP and swizzles; each group's bounds are formed by one
// lane; the codes are code_pair.  The next item's loads are in flight while an item is coded.
constexpr int kPrefillBlocks = 1024;   // 4-wave workgroups: four per CU, one round

__device__ __forceinline__ uint32_t rot16(uint32_t v) { return __builtin_rotateleft32(v, 16); }

// Values: item = 16 destination tokens of one row (half a code tile).  Lane bits 0..5 =
// (e, hh, cb0, p0, p1, a1): tokens 4a..4a+3 of the item with a = 2 a1 + hh, and channels
// 8cb..8cb+7 with cb = 4p + 2e + cb0, i.e. 32p + 16e + 8cb0 + k (k = 0..7).  A token's channel
// group p lies in the four lanes (e, cb0) of one p, hh, a1; the lane e + 2 cb0 = i forms the
// bounds of its four tokens' i-th.  Code byte (channel, four tokens) is the lane's own; tile
// word (chunk 16kg + n, p) takes its four bytes 2hh + e from the lanes (e, hh) of one quad.
// Tokens outside the call's range are loaded from a token inside it and masked out: their
// words are merged into what memory holds, and their (scale, zero) words are not written.
__global__ __launch_bounds__(kBlock) void quantize_v32_kernel(QuantArgs a) {
    const int lane = threadIdx.x & 63;
    const int e = lane & 1, hh = (lane >> 1) & 1, cb0 = (lane >> 2) & 1, p = (lane >> 3) & 3, a1 = lane >> 5;
    const int cb = 4 * p + 2 * e + cb0;
    const int ta = 8 * a1 + 4 * hh;              // the lane's first token inside the item
    const int lo = a.dst_token_off, hi = a.dst_token_off + a.tokens;
    const int blk0 = lo >> 4, blk1 = (hi - 1) >> 4;   // first and last 16-token block of a row
    const int per_row = blk1 - blk0 + 1;
    // items row-major, wave w taking w, w + W, w + 2W, ... (W waves in the grid): the waves
    // in flight read one window of the source at a time (few pages), and the step from one
    // item to the next is a fixed (rows, blocks) increment
    const int64_t W = (int64_t)gridDim.x * (kBlock / 64);
    const int64_t first = (int64_t)blockIdx.x * (kBlock / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (first >= a.rows * (int64_t)per_row) return;
    const int64_t drow = W / per_row;
    const int dblk = (int)(W - drow * per_row);
    int64_t row = first / per_row;
    int blk = blk0 + (int)(first - row * per_row);
    auto load = [&](int64_t r, int b, uint4 (&x)[4]) {   // source token t - lo of row r
        const char* src = reinterpret_cast<const char*>(a.src + r * a.src_row_stride + (int64_t)(b * 16 - lo) * kD);
        const int t0 = b * 16 + ta;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t t = (uint32_t)(std::min(std::max(t0 + j, lo), hi - 1) - b * 16);   // 0..15
            x[j] = *reinterpret_cast<const uint4*>(src + (t * kD + 8 * cb) * 2u);
        }
    };
    const int q = 2 * hh + e;                    // byte of the tile word this lane fills
    const uint32_t sel0 = 0x0C0C0C0Cu & ~(0xFFu << (8 * q));   // byte 0 of a value to byte q
    const uint32_t sel1 = sel0 | (2u << (8 * q));              // byte 2 of a value to byte q
    const int gi = e + 2 * cb0;                  // the token whose bounds this lane forms

    uint4 cur[4];
    load(row, blk, cur);
    for (;;) {
        // the next item (the last one again at the end: the loads are always issued, so the
        // count of loads in flight is fixed)
        int64_t nrow = row + drow;
        int nblk = blk + dblk;
        if (nblk > blk1) {
            nblk -= per_row;
            ++nrow;
        }
        const bool more = nrow < a.rows;
        uint4 nx[4];
        load(more ? nrow : row, more ? nblk : blk, nx);

        const int t0 = blk * 16 + ta;            // destination token of cur[0]
        uint32_t mm[4];                          // minima of tokens (0,1), (2,3); maxima of the same
        {
            uint32_t mn[4], mx[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t m = pk_min(pk_min(cur[j].x, cur[j].y), pk_min(cur[j].z, cur[j].w));
                const uint32_t M = pk_max(pk_max(cur[j].x, cur[j].y), pk_max(cur[j].z, cur[j].w));
                mn[j] = pk_min(m, rot16(m));
                mx[j] = pk_max(M, rot16(M));
            }
            mm[0] = __builtin_amdgcn_perm(mn[1], mn[0], 0x05040100u);
            mm[1] = __builtin_amdgcn_perm(mn[3], mn[2], 0x05040100u);
            mm[2] = __builtin_amdgcn_perm(mx[1], mx[0], 0x05040100u);
            mm[3] = __builtin_amdgcn_perm(mx[3], mx[2], 0x05040100u);
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            mm[n] = pk_min(mm[n], dpp_u<kQuadXor1>(mm[n]));
            mm[n + 2] = pk_max(mm[n + 2], dpp_u<kQuadXor1>(mm[n + 2]));
        }
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            mm[n] = pk_min(mm[n], swz_u<kSwzXor4>(mm[n]));
            mm[n + 2] = pk_max(mm[n + 2], swz_u<kSwzXor4>(mm[n + 2]));
        }
        const uint32_t mnp = (gi >> 1) ? mm[1] : mm[0], mxp = (gi >> 1) ? mm[3] : mm[2];
        const GroupV gb = group_bounds(h2f((gi & 1) ? mnp >> 16 : mnp & 0xffffu),
                                       h2f((gi & 1) ? mxp >> 16 : mxp & 0xffffu));
        {
            const int tg = t0 + gi;
            if (tg >= lo && tg < hi)
                __builtin_nontemporal_store(gb.pair, reinterpret_cast<uint32_t*>(a.v_sz) + value_pair_index<kG>(row * a.token_cap + tg, p));
        }
        // codes; D[m]: the code bytes of channels 8cb + 2m (bits 0..7) and 8cb + 2m + 1 (16..23),
        // token j at bits 2j of each
        const uint32_t w12 = gb.v1 | (gb.v2 << 16), w33 = gb.v3 | (gb.v3 << 16);
        uint32_t D[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // token j's bounds from the lane (e, cb0) = (j & 1, j >> 1) of this group
            constexpr int kQ[2] = {0xA0, 0xF5};
            constexpr int kS[2] = {0x001B, 0x009B};
            uint32_t b12, b33;
            if ((j & 1) == 0) {
                b12 = dpp_u<kQ[0]>(w12);
                b33 = dpp_u<kQ[0]>(w33);
            } else {
                b12 = dpp_u<kQ[1]>(w12);
                b33 = dpp_u<kQ[1]>(w33);
            }
            if ((j >> 1) == 0) {
                b12 = swz_u<kS[0]>(b12);
                b33 = swz_u<kS[0]>(b33);
            } else {
                b12 = swz_u<kS[1]>(b12);
                b33 = swz_u<kS[1]>(b33);
            }
            const uint32_t v1 = __builtin_amdgcn_perm(b12, b12, 0x01000100u);
            const uint32_t v2 = __builtin_amdgcn_perm(b12, b12, 0x03020302u);
            const uint32_t xs[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) D[m] |= code_pair(xs[m], v1, v2, b33) << (2 * j);
        }
        // byte k (channel 8cb + k) of word (chunk 16kg + 8cb0 + k, p): the quad ORs its four
        // bytes, then lane q writes the words k = 2q, 2q + 1
        uint32_t R[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            R[k] = __builtin_amdgcn_perm(0u, D[k >> 1], (k & 1) ? sel1 : sel0);
            R[k] |= dpp_u<kQuadXor1>(R[k]);
            R[k] |= dpp_u<kQuadXor2>(R[k]);
        }
        const uint32_t W0 = q == 0 ? R[0] : (q == 1 ? R[2] : (q == 2 ? R[4] : R[6]));
        const uint32_t W1 = q == 0 ? R[1] : (q == 1 ? R[3] : (q == 2 ? R[5] : R[7]));
        {
            // the word's tokens: block tokens 8a1 .. 8a1 + 7
            const int tw = blk * 16 + 8 * a1;
            uint32_t mask = 0xFFFFFFFFu;
            if (tw < lo || tw + 8 > hi) {
                mask = 0u;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (tw + u >= lo && tw + u < hi) mask |= 0x0303u << (16 * (u >> 2) + 2 * (u & 3));
            }
            const int kg = 2 * (blk & 1) + a1;
            uint32_t* tile = reinterpret_cast<uint32_t*>(a.v_codes + (row * a.token_cap + (int64_t)(blk >> 1) * kG) * kRowBytes);
            uint32_t* w0 = tile + (16 * kg + 8 * cb0 + 2 * q) * 4 + p;
            uint32_t* w1 = w0 + 4;
            if (mask == 0xFFFFFFFFu) {
                __builtin_nontemporal_store(W0, w0);   // streamed: whole 16-byte chunks per instruction
                __builtin_nontemporal_store(W1, w1);
            } else if (mask != 0u) {
                *w0 = (*w0 & ~mask) | (W0 & mask);
                *w1 = (*w1 & ~mask) | (W1 & mask);
            }
        }
        if (!more) break;
        row = nrow;
        blk = nblk;
#pragma unroll
        for (int j = 0; j < 4; ++j) cur[j] = nx[j];
    }
}

// Keys: item = (row, group g): one whole code tile per wave.  Lane bits 0..2 = a, 3..5 = w:
// tokens 4a..4a+3 of the group and channels 16w..16w+15, i.e. tile word w of four tokens.  A
// channel's 32 tokens lie in the eight lanes a of one w; after a reduce-scatter over them
// lane a holds the minimum and maximum of the channel pair 16w + 2r, + 1 with
// r = 4 (a & 1) + 2 ((a >> 1) & 1) + (a >> 2), forms the pair's bounds and passes them through
// LDS to the eight lanes.  Each store instruction writes whole 16-byte chunks of the tile.
__global__ __launch_bounds__(kBlock) void quantize_k32_kernel(QuantArgs a) {
    __shared__ __align__(16) uint32_t sh_v[kBlock / 64][3][kD / 2];   // bounds of channel pairs
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int la = lane & 7, w = lane >> 3;
    const int per_row = a.tokens / kG;
    const int g_first = a.dst_token_off / kG;
    // items row-major, wave w taking w, w + W, ... as in the value quantizer
    const int64_t W = (int64_t)gridDim.x * (kBlock / 64);
    const int64_t first = (int64_t)blockIdx.x * (kBlock / 64) + wave;
    if (first >= a.rows * (int64_t)per_row) return;
    const int64_t drow = W / per_row;
    const int dg = (int)(W - drow * per_row);
    int64_t row = first / per_row;
    int g = (int)(first - row * per_row);        // group - g_first

    auto load = [&](int64_t r, int gg, uint4 (&x)[8]) {
        const char* src = reinterpret_cast<const char*>(a.src + r * a.src_row_stride + (int64_t)gg * kG * kD);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = ((uint32_t)(4 * la + j) * kD + 16 * w) * 2u;
            x[2 * j] = *reinterpret_cast<const uint4*>(src + off);
            x[2 * j + 1] = *reinterpret_cast<const uint4*>(src + off + 16);
        }
    };
    const bool o1 = la & 1, o2 = (la >> 1) & 1, o3 = la >> 2;
    const int r = 4 * (la & 1) + 2 * ((la >> 1) & 1) + (la >> 2);   // the channel pair this lane bounds

    uint4 cur[8];
    load(row, g, cur);
    for (;;) {
        int64_t nrow = row + drow;
        int ng = g + dg;
        if (ng >= per_row) {
            ng -= per_row;
            ++nrow;
        }
        const bool more = nrow < a.rows;
        uint4 nx[8];
        load(more ? nrow : row, more ? ng : g, nx);

        uint32_t xs[4][8];   // token j, channel pair m (16w + 2m, + 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 u = cur[2 * j], v = cur[2 * j + 1];
            xs[j][0] = u.x; xs[j][1] = u.y; xs[j][2] = u.z; xs[j][3] = u.w;
            xs[j][4] = v.x; xs[j][5] = v.y; xs[j][6] = v.z; xs[j][7] = v.w;
        }
        uint32_t MN[8], MX[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            MN[m] = pk_min(pk_min(xs[0][m], xs[1][m]), pk_min(xs[2][m], xs[3][m]));
            MX[m] = pk_max(pk_max(xs[0][m], xs[1][m]), pk_max(xs[2][m], xs[3][m]));
        }
        // reduce-scatter over the eight lanes a: partner a ^ 1 takes pairs 4..7 when a is odd,
        // a ^ 2 then the upper two of the four, a ^ 4 the upper one of the two
        uint32_t mn1[4], mx1[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const uint32_t kn = o1 ? MN[n + 4] : MN[n], sn = o1 ? MN[n] : MN[n + 4];
            const uint32_t kx = o1 ? MX[n + 4] : MX[n], sx = o1 ? MX[n] : MX[n + 4];
            mn1[n] = pk_min(kn, dpp_u<kQuadXor1>(sn));
            mx1[n] = pk_max(kx, dpp_u<kQuadXor1>(sx));
        }
        uint32_t mn2[2], mx2[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const uint32_t kn = o2 ? mn1[n + 2] : mn1[n], sn = o2 ? mn1[n] : mn1[n + 2];
            const uint32_t kx = o2 ? mx1[n + 2] : mx1[n], sx = o2 ? mx1[n] : mx1[n + 2];
            mn2[n] = pk_min(kn, dpp_u<kQuadXor2>(sn));
            mx2[n] = pk_max(kx, dpp_u<kQuadXor2>(sx));
        }
        uint32_t mn3, mx3;
        {
            const uint32_t kn = o3 ? mn2[1] : mn2[0], sn = o3 ? mn2[0] : mn2[1];
            const uint32_t kx = o3 ? mx2[1] : mx2[0], sx = o3 ? mx2[0] : mx2[1];
            mn3 = pk_min(kn, swz_u<kSwzXor4>(sn));
            mx3 = pk_max(kx, swz_u<kSwzXor4>(sx));
        }
        const GroupV b0 = group_bounds(h2f(mn3 & 0xffffu), h2f(mx3 & 0xffffu));
        const GroupV b1 = group_bounds(h2f(mn3 >> 16), h2f(mx3 >> 16));
        const int gd = g_first + g;                // destination group
        *reinterpret_cast<uint2*>(reinterpret_cast<uint32_t*>(a.k_sz) + (row * (a.token_cap / kG) + gd) * kD + 16 * w + 2 * r) =
            make_uint2(b0.pair, b1.pair);
        sh_v[wave][0][8 * w + r] = b0.v1 | (b1.v1 << 16);
        sh_v[wave][1][8 * w + r] = b0.v2 | (b1.v2 << 16);
        sh_v[wave][2][8 * w + r] = b0.v3 | (b1.v3 << 16);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint32_t vb[3][8];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const uint4 lo4 = *reinterpret_cast<const uint4*>(&sh_v[wave][k][8 * w]);
            const uint4 hi4 = *reinterpret_cast<const uint4*>(&sh_v[wave][k][8 * w + 4]);
            vb[k][0] = lo4.x; vb[k][1] = lo4.y; vb[k][2] = lo4.z; vb[k][3] = lo4.w;
            vb[k][4] = hi4.x; vb[k][5] = hi4.y; vb[k][6] = hi4.z; vb[k][7] = hi4.w;
        }
        // tile word w of token 4a + j: channel c = 2m + b at bit 8 (c & 3) + 2 (c >> 2)
        uint8_t* tile = a.k_codes + (row * a.token_cap + (int64_t)gd * kG) * kRowBytes;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t C[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) C[m] = code_pair(xs[j][m], vb[0][m], vb[1][m], vb[2][m]);
            const uint32_t word = __builtin_amdgcn_perm(C[1], C[0], 0x06040200u) |
                                  (__builtin_amdgcn_perm(C[3], C[2], 0x06040200u) << 2) |
                                  (__builtin_amdgcn_perm(C[5], C[4], 0x06040200u) << 4) |
                                  (__builtin_amdgcn_perm(C[7], C[6], 0x06040200u) << 6);
            *reinterpret_cast<uint32_t*>(tile + key_word_offset(4 * la + j, w)) = word;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (!more) break;
        row = nrow;
        g = ng;
#pragma unroll
        for (int j = 0; j < 8; ++j) cur[j] = nx[j];
    }
}

// 4-bit codes: grid.x = rows * (tokens / GS); one key token group per workgroup.
template <int GS>
__global__ __launch_bounds__(kBlock) void quantize_k4_kernel(QuantArgs a) {
    __shared__ uint4 tile4[GS * kD / 8];
    __shared__ float sh_mn[kD], sh_s[kD];
    const int groups = a.tokens / GS;
    const int64_t row = blockIdx.x / groups;
    const int g = blockIdx.x % groups;
    const uint4* s4 = reinterpret_cast<const uint4*>(a.src + row * a.src_row_stride + (int64_t)g * GS * kD);
#pragma unroll
    for (int i = threadIdx.x; i < GS * kD / 8; i += kBlock) tile4[i] = s4[i];
    __syncthreads();
    const int dst_tok = a.dst_token_off + g * GS;
    quant_k4_group<GS>(reinterpret_cast<const uint16_t*>(tile4), sh_mn, sh_s,
                       a.k_codes + (row * a.token_cap + dst_tok) * kRowBytes4,
                       reinterpret_cast<uint32_t*>(a.k_sz) + (row * (a.token_cap / GS) + dst_tok / GS) * kD);
}

// 4-bit codes: grid.x = rows * ceil(tokens / 64); 64 value tokens per workgroup.
template <int GS>
__global__ __launch_bounds__(kBlock) void quantize_v4_kernel(QuantArgs a) {
    const int per_row = (a.tokens + 63) / 64;
    const int64_t row = blockIdx.x / per_row;
    const int base = (int)(blockIdx.x % per_row) * 64;
    const int n = min(64, a.tokens - base);
    const int64_t dst = row * a.token_cap + a.dst_token_off + base;
    quant_v4_tokens<GS>(a.src + row * a.src_row_stride + (int64_t)base * kD, kD, n, a.v_codes + dst * kRowBytes4,
                        reinterpret_cast<uint32_t*>(a.v_sz) + value_pair_index<GS>(dst, 0));
}

// grid.x = ceil(rows * n * 16 / 256): copy tokens [first, first+n) of each row into ring
// slots 0..n-1, keys and values.
__global__ __launch_bounds__(kBlock) void residual_load_kernel(ResidualArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;   // 16-byte chunk index
    const int64_t total = a.rows * (int64_t)a.n * 16;
    if (i >= total) return;
    const int64_t row = i / (a.n * 16);
    const int rem = (int)(i % (a.n * 16));
    const int t = rem >> 4, c = rem & 15;
    const int64_t so = row * a.src_row_stride + (int64_t)(a.first + t) * kD;
    const int64_t d = (row * a.residual_cap + t) * kD;
    reinterpret_cast<uint4*>(a.k_res + d)[c] = reinterpret_cast<const uint4*>(a.k + so)[c];
    reinterpret_cast<uint4*>(a.v_res + d)[c] = reinterpret_cast<const uint4*>(a.v + so)[c];
}

// grid (rows, groups of a flush).  Optional flush of the F ring tokens from flush_slot (F =
// GS, or the whole ring with flush_all) into key groups flush_group.. / value tokens
// flush_group*GS.., one workgroup per group, then the new token into new_slot.  In a ragged
// batch each row takes these from its sequence's state (flush when its ring is full); a
// sequence whose state is out of range, or whose flush would pass token_cap, is skipped and
// flagged.
template <int GS, int BITS>
__global__ __launch_bounds__(kBlock) void append_flush_kernel(AppendArgs a) {
    __shared__ uint4 tile4[GS * kD / 8];
    __shared__ float4 sh_q[kQSlots];   // 2-bit keys: minimum and thresholds; 4-bit: minimum and scale arrays
    float* sh_mn = reinterpret_cast<float*>(sh_q);
    float* sh_s = sh_mn + kD;
    const int64_t row = blockIdx.x;
    const int part = blockIdx.y;   // which group of the flush this workgroup quantizes
    const int tid = threadIdx.x;
    const int F = a.flush_all ? a.residual_cap : GS;   // tokens a flush moves
    int do_flush = a.do_flush, flush_slot = a.flush_slot, flush_group = a.flush_group, new_slot = a.new_slot;
    if (a.seq_state != nullptr) {
        int32_t* s = a.seq_state + 4 * (row / a.kv_heads);
        const int32_t nq = s[0], nr = s[1], rh = s[2];
        const bool ok = state_in_range(nq, nr, rh, a.token_cap, a.residual_cap, GS);
        const bool flush = nr == a.residual_cap;
        if (!ok || (flush && nq + F > a.token_cap)) {   // the whole workgroup leaves together
            if (row % a.kv_heads == 0 && part == 0 && tid == 0)
                __hip_atomic_fetch_or(&s[3], ok ? kSeqCapacity : kSeqBadState, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        do_flush = flush;
        flush_slot = rh;
        flush_group = nq / GS;
        const int head = flush ? (rh + F) % a.residual_cap : rh;
        new_slot = (head + (flush ? nr - F : nr)) % a.residual_cap;
    }
    if (part > 0 && (!do_flush || part * GS >= F)) return;   // (no such group of this row's flush)
    if (do_flush) {
        // group `part` of the flush: GS ring tokens, contiguous (the ring length and its head
        // are multiples of GS)
        const int slot = (flush_slot + part * GS) % a.residual_cap;
        const int group = flush_group + part;
        const uint4* kr = reinterpret_cast<const uint4*>(a.k_res + (row * a.residual_cap + slot) * kD);
#pragma unroll
        for (int i = tid; i < GS * kD / 8; i += kBlock) tile4[i] = kr[i];
        __syncthreads();
        const int dst_tok = group * GS;
        uint32_t* kp = reinterpret_cast<uint32_t*>(a.k_sz) + (row * (a.token_cap / GS) + group) * kD;
        if constexpr (BITS == 4) {
            quant_k4_group<GS>(reinterpret_cast<const uint16_t*>(tile4), sh_mn, sh_s,
                               a.k_codes + (row * a.token_cap + dst_tok) * kRowBytes4, kp);
            quant_v4_tokens<GS>(a.v_res + (row * a.residual_cap + slot) * kD, kD, GS,
                                a.v_codes + (row * a.token_cap + dst_tok) * kRowBytes4,
                                reinterpret_cast<uint32_t*>(a.v_sz) + value_pair_index<GS>(row * a.token_cap + dst_tok, 0));
        } else {
            uint8_t* kc = a.k_codes + row * a.token_cap * kRowBytes + (int64_t)(dst_tok / kG) * kTileBytes;
            quant_k_group<GS>(reinterpret_cast<const uint16_t*>(tile4), sh_q, kc, kp);
            // values: the same GS ring tokens as GS/32 value tiles
            __shared__ __align__(16) uint8_t sh_codes[kG][kD];
#pragma unroll 1
            for (int tl = 0; tl < GS / kG; ++tl)
                quant_v_tile<GS>(a.v_res + (row * a.residual_cap + slot + tl * kG) * kD, kD, 0, kG, sh_codes,
                                 a.v_codes + (row * a.token_cap + dst_tok + tl * kG) * kRowBytes,
                                 reinterpret_cast<uint32_t*>(a.v_sz) +
                                     value_pair_index<GS>(row * a.token_cap + dst_tok + tl * kG, 0));
        }
        __syncthreads();   // every read of the flushed slots is done before the overwrite
    }
    // The new token goes to the first flushed group's first slot (or anywhere in the ring
    // without a flush): part 0 stores it, after its reads of that group.
    if (part == 0 && tid < 32) {
        const int c = tid & 15;
        const uint16_t* src = (tid < 16 ? a.k_new : a.v_new) + row * kD;
        uint16_t* dst = (tid < 16 ? a.k_res : a.v_res) + (row * a.residual_cap + new_slot) * kD;
        reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
    }
}

// Ragged batch, after the appends: one thread per sequence moves its state on by one token
// (and by one flushed group when its ring was full), with the decisions the appends took.
__global__ __launch_bounds__(64) void seq_state_update_kernel(AppendArgs a, int32_t batch) {
    const int64_t b = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (b >= batch) return;
    int32_t* s = a.seq_state + 4 * b;
    const int32_t nq = s[0], nr = s[1], rh = s[2], G = a.group;
    if (!state_in_range(nq, nr, rh, a.token_cap, a.residual_cap, G)) return;
    const bool flush = nr == a.residual_cap;
    const int32_t F = a.flush_all ? a.residual_cap : G;
    if (flush && nq + F > a.token_cap) return;
    s[0] = flush ? nq + F : nq;
    s[1] = (flush ? nr - F : nr) + 1;
    s[2] = flush ? (rh + F) % a.residual_cap : rh;
}

// ------------------------------------------------------------------ launchers ----

hipError_t launch_quantize_k(const QuantArgs& a, hipStream_t s) {
    const int64_t blocks = a.rows * (int64_t)(a.tokens / a.group);
    if (blocks == 0) return hipSuccess;
    if (a.bits == 4) {
        KIVI_BY_GROUP(a.group, hipLaunchKernelGGL(quantize_k4_kernel<GS>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a))
    } else if (a.group == kG) {
        const int64_t waves = blocks;   // items: (row, group)
        hipLaunchKernelGGL(quantize_k32_kernel, dim3((unsigned)std::min<int64_t>((waves + 3) / 4, kPrefillBlocks)),
                           dim3(kBlock), 0, s, a);
    } else {
        KIVI_BY_GROUP(a.group, hipLaunchKernelGGL(quantize_k_kernel<GS>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a))
    }
    return hipGetLastError();
}

hipError_t launch_quantize_v(const QuantArgs& a, hipStream_t s) {
    if (a.tokens <= 0) return hipSuccess;
    if (a.bits == 4) {
        const int64_t blocks4 = a.rows * (int64_t)((a.tokens + 63) / 64);
        KIVI_BY_GROUP(a.group, hipLaunchKernelGGL(quantize_v4_kernel<GS>, dim3((unsigned)blocks4), dim3(kBlock), 0, s, a))
        return hipGetLastError();
    }
    if (a.group == kG) {   // items: 16 destination tokens of a row
        const int64_t per_row = (a.dst_token_off + a.tokens - 1) / 16 - a.dst_token_off / 16 + 1;
        const int64_t waves = a.rows * per_row;
        if (waves == 0) return hipSuccess;
        hipLaunchKernelGGL(quantize_v32_kernel, dim3((unsigned)std::min<int64_t>((waves + 3) / 4, kPrefillBlocks)),
                           dim3(kBlock), 0, s, a);
        return hipGetLastError();
    }
    const int64_t n_tiles = (a.dst_token_off + a.tokens - 1) / kG - a.dst_token_off / kG + 1;
    const int64_t blocks = a.rows * n_tiles;
    if (blocks == 0) return hipSuccess;
    KIVI_BY_GROUP(a.group, hipLaunchKernelGGL(quantize_v_kernel<GS>, dim3((unsigned)blocks), dim3(kBlock), 0, s, a))
    return hipGetLastError();
}

hipError_t launch_residual_load(const ResidualArgs& a, hipStream_t s) {
    const int64_t blocks = (a.rows * (int64_t)a.n * 16 + kBlock - 1) / kBlock;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(residual_load_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

// grid (rows, groups of the flush): a flush of the whole residual quantizes its R/G groups
// in parallel
hipError_t launch_append_flush(const AppendArgs& a, hipStream_t s) {
    const unsigned parts = a.do_flush && a.flush_all ? (unsigned)(a.residual_cap / a.group) : 1u;
    const dim3 grid((unsigned)a.rows, parts);
    if (a.bits == 4) {
        KIVI_BY_GROUP(a.group, hipLaunchKernelGGL((append_flush_kernel<GS, 4>), grid, dim3(kBlock), 0, s, a))
    } else {
        KIVI_BY_GROUP(a.group, hipLaunchKernelGGL((append_flush_kernel<GS, 2>), grid, dim3(kBlock), 0, s, a))
    }
    return hipGetLastError();
}

hipError_t launch_append_flush_ragged(const AppendArgs& a, int32_t batch, hipStream_t s) {
    const unsigned parts = a.flush_all ? (unsigned)(a.residual_cap / a.group) : 1u;
    const dim3 grid((unsigned)a.rows, parts);
    if (a.bits == 4) {
        KIVI_BY_GROUP(a.group, hipLaunchKernelGGL((append_flush_kernel<GS, 4>), grid, dim3(kBlock), 0, s, a))
    } else {
        KIVI_BY_GROUP(a.group, hipLaunchKernelGGL((append_flush_kernel<GS, 2>), grid, dim3(kBlock), 0, s, a))
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(seq_state_update_kernel, dim3((unsigned)((batch + 63) / 64)), dim3(64), 0, s, a, batch);
    return hipGetLastError();
}

}  // namespace kivi
