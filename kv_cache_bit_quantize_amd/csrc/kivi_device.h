// kivi_device.h -- device-side building blocks shared by the libkivi kernels (gfx950).
//
// Layout and quantizer are those declared in include/kivi.h.  This header is part of the
// HIP library only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kivi {

constexpr int kD = 128;             // head_dim implemented here
constexpr int kG = 32;              // group size (tokens for keys, channels for values)
constexpr int kRowBytes = kD / 4;   // packed code bytes per token
constexpr int kBlock = 256;         // threads per workgroup (4 wave64)

__device__ __forceinline__ float h2f(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f2h(float f) {   // v_cvt_f16_f32: RNE, subnormals kept
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---------------------------------------------------------------------------------
// Asymmetric 2-bit group quantizer (KIVI title, "asymmetric 2bit"; record "Methodology").
// zero = min, scale = fp16(fp32(max - min) / 3), both with signed zeros read as +0;
// code = clamp(rne(fp32(x - min) / scale), 0, 3), 0 when the stored scale is 0.
// Every operation is one IEEE binary32 operation: no contraction, true division.
// ---------------------------------------------------------------------------------
struct GroupQ {
    float mn;     // zero point (canonical +0)
    float s;      // stored fp16 scale, widened
    uint32_t pair;  // fp16 scale in bits 0..15, fp16 zero in bits 16..31 (memory order)
};

__device__ __forceinline__ GroupQ group_params(float mn, float mx) {
#pragma clang fp contract(off)
    GroupQ q;
    mn = mn + 0.0f;                 // -0 + +0 = +0 under round-to-nearest
    mx = mx + 0.0f;
    float range = mx - mn;
    float s32 = range / 3.0f;
    uint32_t sh = f2h(s32);
    q.mn = mn;
    q.s = h2f(sh);
    q.pair = sh | (f2h(mn) << 16);
    return q;
}

__device__ __forceinline__ uint32_t code_of(float x, const GroupQ& q) {
#pragma clang fp contract(off)
    if (q.s == 0.0f) return 0u;
    float d = x - q.mn;
    float t = d / q.s;
    float r = __builtin_rintf(t);   // v_rndne_f32: ties to even
    r = __builtin_fminf(r, 3.0f);
    return (uint32_t)r;
}

// wave64 cross-lane helpers (ds_swizzle/DPP chosen by the compiler for __shfl_xor)
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
