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
