// kivi_device.h -- device-side building blocks shared by the libkivi kernels (gfx950).
//
// Layout and quantizer are those declared in include/kivi.h.  This header is part of the
// HIP library only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kivi {

constexpr int kD = 128;             // head_dim implemented here
constexpr int kG = 32;              // tokens per packed code tile, and the smallest group size
// Group sizes (tokens per key group, channels per value group) the kernels are built for.
__host__ __device__ constexpr bool group_supported(int g) { return g == 32 || g == 64 || g == 128; }
// Launch code: one template instance per supported group size (GS inside CALL).
#define KIVI_BY_GROUP(G, CALL)                  \
    switch (G) {                                \
        case 32: { constexpr int GS = 32; CALL; break; }   \
        case 64: { constexpr int GS = 64; CALL; break; }   \
        case 128: { constexpr int GS = 128; CALL; break; } \
        default: return hipErrorInvalidValue;   \
    }

constexpr int kRowBytes = kD / 4;   // packed code bytes per token (2-bit codes)
constexpr int kRowBytes4 = kD / 2;  // 4-bit codes: token-major, channel j in byte j/2 (even channel low)
constexpr int kBlock = 256;         // threads per workgroup (4 wave64)

// Packed code layout (include/kivi.h).  A row holds one 1024-byte tile per 32-token group.
//  * Key tiles: the 16 channels 16w..16w+15 of a token form one 32-bit word, channel offset
//    c = 4i + b (0..15) in byte b at bits 2i..2i+1, i.e. at bit 8b + 2i, so masking a word
//    with 0x03030303 << 2i leaves the codes of channels 4i..4i+3, one per byte.  16-byte
//    chunk (16k + n) holds words k, 4+k of token n, then of token 16+n: lane 16k + n of a
//    wave loading chunk (lane) reads the whole tile in one contiguous access and gets
//    exactly its part of the integer matrix instruction's K x N operand (channels
//    16k..16k+15 and 64+16k.. of tokens n and 16+n).
//  * Value tiles: a byte holds one channel's codes for four consecutive tokens (token 4a+i
//    at bits 2i..2i+1).  16-byte chunk (16k + n) covers tokens 8k..8k+7 and the channels
//    n + 16v; its 32-bit word p holds, byte by byte, channel n+32p for tokens 8k..8k+3,
//    channel n+32p+16 for the same tokens, then both channels for tokens 8k+4..8k+7.  Lane
//    16k + n loading chunk (lane) gets its part of the fp16 matrix instruction's K x N
//    operand (tokens 8k..8k+7 of channels n + 16v) for all eight 16-channel blocks v.
__host__ __device__ constexpr int code_bit(int c) { return 8 * (c & 3) + 2 * (c >> 2); }
constexpr int kTileBytes = kG * kD / 4;     // 1024

// byte offset, inside a row, of word w (0..7) of key token t
__host__ __device__ constexpr int64_t key_word_offset(int64_t t, int w) {
    return (t >> 5) * kTileBytes + ((w & 3) * 16 + (t & 15)) * 16 + ((t >> 4) & 1) * 8 + (w >> 2) * 4;
}
// index (in 32-bit pairs), inside a row, of the value (scale, zero) of token t, group k
// (groups of GS channels: kD / GS pairs per token)
template <int GS = kG>
__host__ __device__ constexpr int64_t value_pair_index(int64_t t, int k) { return t * (kD / GS) + k; }

// A cache state the kernels can use without reading outside the buffers: whole groups in the
// history, within capacity, and a ring head on a group boundary (group: tokens per key group).
__host__ __device__ inline bool state_in_range(int32_t n_quant, int32_t n_res, int32_t res_head, int32_t token_cap,
                                               int32_t residual_cap, int32_t group) {
    return n_quant >= 0 && n_quant <= token_cap && n_quant % group == 0 && n_res >= 0 && n_res <= residual_cap &&
           res_head >= 0 && res_head < residual_cap && res_head % group == 0;
}

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f2h(float f) {   // v_cvt_f16_f32: RNE, subnormals kept
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Loads with the non-temporal hint, for cache streams read once per call.  They pay where each
// load instruction reads whole cache lines: the 2-bit single-query and uniform query-group
// attention (the long-context call 11% faster) and the 4-bit attention (once its loads read
// whole rows: 11% faster).  Where a line is split between instructions the hint lets it go
// before the second one and the line is read twice: the pre-RoPE, fp16 and ragged kernels and
// the prefill quantizers measured slower with it and keep plain loads (the pre-RoPE kernel's
// query-group calls also re-read a kv head from several workgroups).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_nt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 stream_load16(const void* p) {
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 stream_load8(const void* p) {
    const u32x2_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t stream_load4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// ---------------------------------------------------------------------------------
// Asymmetric 2-bit group quantizer (KIVI title, "asymmetric 2bit"; record "Methodology").
// zero = min, scale = fp16(fp32(max - min) / 3), both with signed zeros read as +0;
// code = clamp(rne(fp32(x - min) / scale), 0, 3), 0 when the stored scale is 0.  The 4-bit
// member of the family divides by 15 and clamps at 15.
// Every operation is one IEEE binary32 operation: no contraction, true division.
// ---------------------------------------------------------------------------------
struct GroupQ {
    float mn;     // zero point (canonical +0)
    float s;      // stored fp16 scale, widened
    uint32_t pair;  // fp16 scale in bits 0..15, fp16 zero in bits 16..31 (memory order)
};

// TOP: the highest code, 3 for 2-bit codes, 15 for 4-bit codes (the same rules otherwise)
template <int TOP = 3>
__device__ __forceinline__ GroupQ group_params(float mn, float mx) {
#pragma clang fp contract(off)
    GroupQ q;
    mn = mn + 0.0f;                 // -0 + +0 = +0 under round-to-nearest
    mx = mx + 0.0f;
    float range = mx - mn;
    float s32 = range / (float)TOP;
    uint32_t sh = f2h(s32);
    q.mn = mn;
    q.s = h2f(sh);
    q.pair = sh | (f2h(mn) << 16);
    return q;
}

template <int TOP = 3>
__device__ __forceinline__ uint32_t code_of(float x, const GroupQ& q) {
#pragma clang fp contract(off)
    if (q.s == 0.0f) return 0u;
    float d = x - q.mn;
    float t = d / q.s;
    float r = __builtin_rintf(t);   // v_rndne_f32: ties to even
    r = __builtin_fminf(r, (float)TOP);
    return (uint32_t)r;
}

// Cross-lane exchange without LDS traffic: DPP for partners inside a 16-lane row
// (quad_perm for lane^1 and lane^2; after those, every lane of a quad holds the same value,
// so the half-row mirror and the row mirror pair each quad / half-row with the other one),
// ds_swizzle for lane^16 and readlane for the two halves of the wave.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// The same move for a pattern in which every lane has a source lane (quad_perm, the mirrors):
// no lane keeps its old value, so none is set up first.
template <int CTRL>
__device__ __forceinline__ float perm_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t perm_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// IEEE 754 maximum (a NaN operand gives NaN).  Unlike fmaxf, which must first quiet a
// signalling NaN in each operand that does not come straight from arithmetic (an extra
// v_max_f32 x, x, x per cross-lane move), it is one v_maximum3_f32.
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// 2^x by the hardware exponential alone (v_exp_f32).  exp2f adds a range reduction (a
// compare, two selects, an add and a scale) so that results below 2^-126 come out as
// subnormals; here they are zero.  Every use is a softmax weight or rescale factor relative
// to the running maximum, where a factor below 2^-126 is far under the output's resolution.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float xor1_f(float v) { return dpp_f<0xB1>(v); }    // quad_perm [1,0,3,2]
__device__ __forceinline__ float xor2_f(float v) { return dpp_f<0x4E>(v); }    // quad_perm [2,3,0,1]
__device__ __forceinline__ float hmirror_f(float v) { return dpp_f<0x141>(v); } // lane i <-> 7-i in 8
__device__ __forceinline__ float mirror_f(float v) { return dpp_f<0x140>(v); }  // lane i <-> 15-i in 16
__device__ __forceinline__ float xor16_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
__device__ __forceinline__ float ror4_f(float v) { return dpp_f<0x124>(v); }   // lane (i+4)%16 of the row
__device__ __forceinline__ float ror8_f(float v) { return dpp_f<0x128>(v); }   // lane (i+8)%16 of the row
// Sums over the 32 lanes of each half-wave of four values at once: afterwards the lane with
// bits (b0, b1) = (lane & 1, (lane >> 1) & 1) holds the sum of v[2*b0 + b1].  Lanes first
// exchange halves of their sets (lane^1, then lane^2), then sum the rest over lanes that
// agree in their two low bits (row rotations by 4 and 8, then lane^16).
__device__ __forceinline__ float half_sum4(const float (&v)[4]) {
    const int lane = threadIdx.x & 63;
    const bool b0 = lane & 1, b1 = lane & 2;
    const float k0 = b0 ? v[2] : v[0], k1 = b0 ? v[3] : v[1];
    const float s0 = b0 ? v[0] : v[2], s1 = b0 ? v[1] : v[3];
    const float u0 = k0 + xor1_f(s0), u1 = k1 + xor1_f(s1);
    const float kk = b1 ? u1 : u0, ss = b1 ? u0 : u1;
    float x = kk + xor2_f(ss);
    x += ror4_f(x);
    x += ror8_f(x);
    return x + xor16_f(x);
}
// sum / max over the 32 lanes of each half-wave (every lane gets its half's result)
__device__ __forceinline__ float half_sum(float v) {
    v += xor1_f(v);
    v += xor2_f(v);
    v += hmirror_f(v);
    v += mirror_f(v);
    return v + xor16_f(v);
}
__device__ __forceinline__ float half_max(float v) {
    v = fmax_ieee(v, perm_f<0xB1>(v));
    v = fmax_ieee(v, perm_f<0x4E>(v));
    v = fmax_ieee(v, perm_f<0x141>(v));
    v = fmax_ieee(v, perm_f<0x140>(v));
    return fmax_ieee(v, xor16_f(v));
}
// half_max for values that are never negative: their bit patterns order as unsigned
// integers do, and an integer maximum takes its cross-lane operand directly (one
// v_max_u32 with a DPP source per step)
__device__ __forceinline__ float half_max_nonneg(float f) {
    uint32_t v = __builtin_bit_cast(uint32_t, f);
    v = max(v, perm_u<0xB1>(v));
    v = max(v, perm_u<0x4E>(v));
    v = max(v, perm_u<0x141>(v));
    v = max(v, perm_u<0x140>(v));
    v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
    return __builtin_bit_cast(float, v);
}
// max over lanes that differ in bits 2..5, for values already equal inside each quad;
// the result is wave-uniform
__device__ __forceinline__ float wave_max_quads(float v) {
    v = __builtin_fmaxf(v, hmirror_f(v));
    v = __builtin_fmaxf(v, mirror_f(v));
    v = __builtin_fmaxf(v, xor16_f(v));
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return __builtin_fmaxf(lo, hi);
}
// sum over the 4 lanes of a quad
__device__ __forceinline__ float quad_sum(float v) {
    v += xor1_f(v);
    return v + xor2_f(v);
}

// wave64 cross-lane helpers through ds_bpermute (outside the hot loops)
__device__ __forceinline__ float wave_max_xor(float v, int from, int to) {
    for (int m = from; m <= to; m <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_min_xor(float v, int from, int to) {
    for (int m = from; m <= to; m <<= 1) v = __builtin_fminf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_sum_xor(float v, int from, int to) {
    for (int m = from; m <= to; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace kivi
