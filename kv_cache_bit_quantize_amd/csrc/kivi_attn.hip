// kivi_attn.hip -- fused decode attention over the 2-bit cache (gfx950).
//
// One query per head attends over the dequantized history followed by the fp16
// residual: out = softmax(sm_scale * q.K^T) . V (error judged at the attention output:
// article "Your KV cache doesn't have a bit problem...", paragraph 3).
//
// Work split: grid (splits, B*Hq).  A 256-thread workgroup owns one query row and a
// contiguous range of key groups; each of its 4 waves walks a quarter of that range
// with its own online softmax (log2 domain).  The waves merge in LDS, the workgroup
// writes one partial (o[128], m, l), and the last workgroup of the row to arrive
// (device-scope arrival counter) merges the row's partials with the log-sum-exp merge
// and writes the output, so one launch does the whole call.  The split holding the last
// groups also reads the fp16 residual.
//
// Inner loop (one wave-iteration = two 32-token key groups, one per half-wave).
// Lane = 32*gh + 4*tq + qq owns tokens 4tq..4tq+3 of group gh and channels
// [32qq, 32qq+32).  Codes are 2 bits, so the loop is bound by HBM and by the vector
// instructions that turn codes into products; it is arranged to need few of them:
//
//  * keys, per token group g: q.(z + c*s) = q.z + (q*s).c.  The 32 lanes of a half
//    compute q*s for 4 channels each, convert it to a 30-bit fixed-point integer with a
//    per-group exponent, split it into four signed bytes, byte-transpose so that one
//    32-bit word holds one byte position of four consecutive channels, and store those
//    words in LDS once.  A token's code word masked with 0x03030303 << 2i gives the codes
//    of channels 4i..4i+3 as bytes (layout in kivi_device.h), so the dot products are
//    exact v_dot4_i32_i8 operations against those words (the per-class factor 4^i of the
//    unshifted masks is divided out of the fixed-point values beforehand).
//  * values, per token: p*(z + c*s) = p*z + (p*s)*c.  v_perm pairs two tokens' code
//    bytes into one word, each code is placed at bits 8-9 or 6-7 of an fp16 whose
//    exponent reads 1.0 (one shift + v_and_or_b32), giving the exact half 1 + c/4 or
//    1 + c/16, and v_dot2_f32_f16 accumulates two tokens per instruction against fp16
//    weights 4*p*s or 16*p*s (kept in range by a power-of-two factor).  The constant
//    part, sum of the weights, is accumulated separately and subtracted at the end.
#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

constexpr int kWaves = kBlock / 64;
constexpr int kPart = kD + 2;   // floats per partial: o[128], m, l
// LDS table of one (parity, wave): two groups' digit planes, then a zero plane
constexpr int kGroupTbl = 4 * kD;             // 4 digit planes of 128 channel bytes
constexpr int kZeroPlane = 2 * kGroupTbl;
constexpr int kTblBytes = kZeroPlane + kD;

typedef int v4i __attribute__((ext_vector_type(4)));

// value of lane 4*(lane/4) + i, for CTRL = quad_perm [i, i, i, i]
template <int CTRL>
__device__ __forceinline__ float quad_bcast(float v) { return dpp_f<CTRL>(v); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }

// (x & m) | o in one instruction (v_and_or_b32 takes its constants in VGPRs)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(o));
    return r;
}

__device__ __forceinline__ float fdot2(uint32_t a, half2_t b, float c) {
    return __builtin_amdgcn_fdot2(as_h2(a), b, c, false);
}

__device__ __forceinline__ void load_q32(const uint16_t* q, float scale, float (&qv)[32]) {
    const uint4* qp = reinterpret_cast<const uint4*>(q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 x = qp[i];
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            qv[8 * i + 2 * k] = h2f(w[k] & 0xffffu) * scale;
            qv[8 * i + 2 * k + 1] = h2f(w[k] >> 16) * scale;
        }
    }
}

// Split partials cross workgroups, which may sit on different XCDs with separate L2 caches.
// They are written and read with agent-scope atomic accesses (global_store / global_load with
// the sc1 coherence bit), each coherent by itself.  Device-scope fences are avoided on
// purpose: on this chip each one writes back and invalidates the whole L2 of the XCD, which
// stalls every other workgroup streaming through it.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt with vmcnt(0) and the other counters left free (expcnt 7, lgkmcnt 15)
constexpr int kWaitVmcnt0 = 0x0F70;

// Log-sum-exp merge of one query row's split partials by the whole workgroup: the m and l of
// every split are read once (spread over the threads), then each output channel sums its
// splits' o with several loads in flight.  out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// lse = (M + log2 L) ln 2.  Re-arms the row counter.
__device__ __forceinline__ void merge_row(const AttnArgs& a, int64_t qrow) {
    __shared__ float sh_sc[kMaxSplits];
    __shared__ float sh_red[kWaves];
    __shared__ float sh_half[2][kD];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float* rowp = a.ws + qrow * kPart;
    const int64_t stride = a.q_rows * kPart;
    float mloc = -INFINITY;
    for (int s = t; s < a.splits; s += kBlock) {
        const float ms = load_coherent(rowp + s * stride + kD);
        sh_sc[s] = ms;
        mloc = fmaxf(mloc, ms);
    }
    mloc = wave_max_xor(mloc, 1, 32);
    if (lane == 0) sh_red[wave] = mloc;
    __syncthreads();
    float M = sh_red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh_red[w]);
    __syncthreads();
    float lloc = 0.0f;
    for (int s = t; s < a.splits; s += kBlock) {
        const float ms = sh_sc[s];
        const float sc = ms == -INFINITY ? 0.0f : exp2f(ms - M);
        sh_sc[s] = sc;
        lloc = fmaf(load_coherent(rowp + s * stride + kD + 1), sc, lloc);
    }
    lloc = wave_sum_xor(lloc, 1, 32);
    if (lane == 0) sh_red[wave] = lloc;
    __syncthreads();
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) L += sh_red[w];
    const int j = t & (kD - 1), h = t >> 7;
    float O = 0.0f;
#pragma unroll 8
    for (int s = h; s < a.splits; s += 2) O = fmaf(load_coherent(rowp + s * stride + j), sh_sc[s], O);
    sh_half[h][j] = O;
    __syncthreads();
    if (t < kD) {
        a.out[qrow * kD + t] = (uint16_t)f2h((sh_half[0][t] + sh_half[1][t]) / L);
        if (t == 0) {
            if (a.lse != nullptr) a.lse[qrow] = (M + log2f(L)) * 0.69314718055994531f;
            a.counters[qrow] = 0u;
        }
    }
}

__global__ __launch_bounds__(kBlock) void attn_split_kernel(AttnArgs a) {
    // Per (parity, wave): the fixed-point digits of q*s for the wave's two groups, as
    // [group][digit plane d][128 channels] bytes, then one all-zero plane.
    __shared__ __align__(16) uint8_t sh_tbl[2][kWaves][kTblBytes];
    __shared__ float sh_o[kWaves][kD];
    __shared__ float sh_m[kWaves], sh_l[kWaves];

    const int split = blockIdx.x;
    const int64_t qrow = blockIdx.y;
    const int64_t b = qrow / a.q_heads;
    const int hq = (int)(qrow % a.q_heads);
    const int64_t kvrow = b * a.kv_heads + hq / a.ratio;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gh = lane >> 5;          // group of the wave-iteration this lane serves
    const int tq = (lane >> 2) & 7, qq = lane & 3;   // value role: tokens 4tq.., channel group qq
    const int wl = lane & 31;          // fixed-point writer role: channels 4wl .. 4wl+3
    const int wk = wl & 3;             // their position i inside the 16-channel block
    const int mrow = lane & 15, kgrp = lane >> 4;     // matrix-operand role

    // query channels 4wl..4wl+3 in the log2 domain
    float qw[4];
    {
        const uint2 x = *reinterpret_cast<const uint2*>(a.q + qrow * kD + 4 * wl);
        qw[0] = h2f(x.x & 0xffffu) * a.sm_log2;
        qw[1] = h2f(x.x >> 16) * a.sm_log2;
        qw[2] = h2f(x.y & 0xffffu) * a.sm_log2;
        qw[3] = h2f(x.y >> 16) * a.sm_log2;
    }
    // codes of channels 4i..4i+3 arrive multiplied by 1, 4, 16, 16 (i = 0..3)
    const float cls_div = wk == 0 ? 1.0f : (wk == 1 ? 0.25f : 0.0625f);

    // A operand of tile t (rows 4t..4t+3 = digits 0..3 of its group, all other rows zero):
    // this lane's 16 bytes come from its own digit plane or from the zero plane.
    int a_off[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        a_off[t] = ((mrow >> 2) == t) ? (t >> 1) * kGroupTbl + (mrow & 3) * kD + 16 * kgrp : kZeroPlane + 16 * kgrp;
    // the zero planes of both parities, written once
    reinterpret_cast<uint32_t*>(&sh_tbl[lane >> 5][wave][kZeroPlane])[lane & 31] = 0u;

    float acc[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) acc[c] = 0.0f;
    float b6 = 0.0f, b8 = 0.0f;        // sums of the fp16 weights of the two value classes
    float zacc = 0.0f, lsum = 0.0f, m = -INFINITY;
    float vs = 0.0f;                   // power-of-two factor keeping the value weights in fp16 range

    const int n_groups = a.n_quant / kG;
    const int g_lo = split * a.groups_per_split;
    const int g_hi = min(n_groups, g_lo + a.groups_per_split);
    const int cnt = max(0, g_hi - g_lo);
    const int per_wave = (cnt + kWaves - 1) / kWaves;
    const int gb = g_lo + min(cnt, wave * per_wave);
    const int ge = g_lo + min(cnt, (wave + 1) * per_wave);
    const int iters = (ge - gb + 1) >> 1;

    const int64_t tok_base = kvrow * (int64_t)a.token_cap;
    const uint8_t* kc_row = a.k_codes + tok_base * kRowBytes;
    const uint8_t* vc_row = a.v_codes + tok_base * kRowBytes;
    const uint32_t* kp_row = reinterpret_cast<const uint32_t*>(a.k_sz) + kvrow * (int64_t)(a.token_cap / kG) * kD;
    const uint32_t* vp_row = reinterpret_cast<const uint32_t*>(a.v_sz) + tok_base * (kD / kG);

    const uint32_t kM6 = 0x00C000C0u, kM8 = 0x03000300u, kOne = 0x3C003C00u;
    const half2_t ones = as_h2(kOne);

    // one wave-iteration's global loads (issued one iteration ahead of their use)
    struct Loads {
        uint4 kp;          // (scale, zero) of key channels 4wl..4wl+3 of group gh
        uint4 kc[2];       // key tile chunk `lane` of both groups (matrix operand B)
        uint2 vw[4];       // value codes of tokens 4tq..4tq+3, channel quarter qq, group gh
        uint32_t vp[4];    // (scale, zero) of the value channel group qq of those tokens
    };
    auto load_iter = [&](int it) {
        Loads L;
        const int g0 = gb + 2 * it;
        const int g1 = g0 + 1 < ge ? g0 + 1 : gb;     // in-bounds address for an idle half
        const int gc = gh ? g1 : g0;
        L.kp = *reinterpret_cast<const uint4*>(kp_row + (int64_t)gc * kD + 4 * wl);
        L.kc[0] = reinterpret_cast<const uint4*>(kc_row + (int64_t)g0 * kTileBytes)[lane];
        L.kc[1] = reinterpret_cast<const uint4*>(kc_row + (int64_t)g1 * kTileBytes)[lane];
        // value tile chunks wl and 32 + wl of group gc hold quarter qq of tokens 4tq..4tq+3
        const uint4* vt = reinterpret_cast<const uint4*>(vc_row + (int64_t)gc * kTileBytes);
        const uint4 v0 = vt[wl], v1 = vt[32 + wl];
        L.vw[0] = make_uint2(v0.x, v0.y);
        L.vw[1] = make_uint2(v0.z, v0.w);
        L.vw[2] = make_uint2(v1.x, v1.y);
        L.vw[3] = make_uint2(v1.z, v1.w);
        const uint4 p = *reinterpret_cast<const uint4*>(vp_row + value_pair_index((int64_t)gc * kG + 4 * tq, qq));
        L.vp[0] = p.x;
        L.vp[1] = p.y;
        L.vp[2] = p.z;
        L.vp[3] = p.w;
        return L;
    };

    Loads cur;
    if (iters > 0) cur = load_iter(0);
    for (int it = 0; it < iters; ++it) {
        const Loads nxt = load_iter(it + 1 < iters ? it + 1 : it);
        const bool gvalid = gb + 2 * it + gh < ge;
        uint8_t* tbl = &sh_tbl[it & 1][wave][0];

        // ---- q*s of this half's group as 30-bit fixed point, four signed byte digits,
        // stored as digit planes
        const uint32_t pr[4] = {cur.kp.x, cur.kp.y, cur.kp.z, cur.kp.w};
        float qs[4], az = 0.0f, mx = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qs[i] = qw[i] * h2f(pr[i] & 0xffffu);
            az = fmaf(qw[i], h2f(pr[i] >> 16), az);
            mx = fmaxf(mx, fabsf(qs[i]));
        }
        az = half_sum(az);
        mx = half_max(mx);
        const int sh = 29 - __builtin_amdgcn_frexp_expf(mx);   // |q*s| * 2^sh < 2^29
        uint32_t dg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qi = (int)__builtin_rintf(__builtin_ldexpf(qs[i] * cls_div, sh));
            dg[i] = ((uint32_t)qi + 0x80808080u) ^ 0x80808080u;    // four signed base-256 digits
        }
        {
            const uint32_t A = __builtin_amdgcn_perm(dg[1], dg[0], 0x05010400u);
            const uint32_t B = __builtin_amdgcn_perm(dg[1], dg[0], 0x07030602u);
            const uint32_t C = __builtin_amdgcn_perm(dg[3], dg[2], 0x05010400u);
            const uint32_t E = __builtin_amdgcn_perm(dg[3], dg[2], 0x07030602u);
            uint32_t* plane = reinterpret_cast<uint32_t*>(tbl + gh * kGroupTbl) + wl;
            plane[0 * kD / 4] = __builtin_amdgcn_perm(C, A, 0x05040100u);   // digit 0 of the 4 channels
            plane[1 * kD / 4] = __builtin_amdgcn_perm(C, A, 0x07060302u);   // digit 1
            plane[2 * kD / 4] = __builtin_amdgcn_perm(E, B, 0x05040100u);   // digit 2
            plane[3 * kD / 4] = __builtin_amdgcn_perm(E, B, 0x07060302u);   // digit 3
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- key logits on the matrix cores: tile t = 2*group + token half, K = 64
        // channels per instruction.  Row 4t + d of the accumulator collects digit d's dot
        // product for tile t's 16 tokens, so lane L ends with the four digit sums of token L.
        v4i cacc = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 kc = cur.kc[t >> 1];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const uint32_t x = (t & 1) ? (kh ? kc.w : kc.z) : (kh ? kc.y : kc.x);
                const v4i bop = {(int)(x & 0x03030303u), (int)(x & 0x0C0C0C0Cu), (int)(x & 0x30303030u),
                                 (int)((x >> 2) & 0x30303030u)};
                const v4i aop = *reinterpret_cast<const v4i*>(tbl + a_off[t] + 64 * kh);
                cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, cacc, 0, 0, 0);
            }
        }
        float lg;
        {
            const int hi = cacc[3] * 256 + cacc[2], lo = cacc[1] * 256 + cacc[0];
            const float tot = fmaf((float)hi, 65536.0f, (float)lo);
            lg = gvalid ? fmaf(tot, __builtin_ldexpf(1.0f, -sh), az) : -INFINITY;
        }

        // ---- online softmax over the wave's 64 tokens (rescale only when the max rises)
        float mloc = half_max(lg);
        mloc = fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mloc), 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mloc), 32)));
        if (mloc > m) {
            const float al = exp2f(m - mloc);
#pragma unroll
            for (int c = 0; c < 32; ++c) acc[c] *= al;
            b6 *= al;
            b8 *= al;
            zacc *= al;
            lsum *= al;
            m = mloc;
        }
        const float pt = exp2f(lg - m);      // this lane's token
        lsum += pt;
        // value role: the weights of tokens 4tq..4tq+3 sit in this lane's quad
        const float p[4] = {quad_bcast<0x00>(pt), quad_bcast<0x55>(pt), quad_bcast<0xAA>(pt), quad_bcast<0xFF>(pt)};
        float w[4], smax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = h2f(cur.vp[i] & 0xffffu);
            w[i] = p[i] * s;
            zacc = fmaf(p[i], h2f(cur.vp[i] >> 16), zacc);
            smax = fmaxf(smax, s);
        }
        const uint2* vw = cur.vw;
        // value weights 16*w*vs must stay below 2^15: shrink vs (a power of two) if needed
        if (__builtin_amdgcn_ballot_w64(smax * vs > 2048.0f || vs == 0.0f)) {
            const float gm = wave_max_xor(smax, 1, 32);
            const float nvs = __builtin_ldexpf(1.0f, 11 - __builtin_amdgcn_frexp_expf(gm));
            if (vs != 0.0f && nvs < vs) {
                const float r = nvs / vs;
#pragma unroll
                for (int c = 0; c < 32; ++c) acc[c] *= r;
                b6 *= r;
                b8 *= r;
            }
            if (vs == 0.0f || nvs < vs) vs = nvs;
        }

        // ---- P.V over the codes: two tokens per v_dot2 against fp16 weights
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            half2_t u6, u8;
            u6.x = (_Float16)(w[2 * pp] * (16.0f * vs));
            u6.y = (_Float16)(w[2 * pp + 1] * (16.0f * vs));
            u8.x = (_Float16)(w[2 * pp] * (4.0f * vs));
            u8.y = (_Float16)(w[2 * pp + 1] * (4.0f * vs));
            b6 = __builtin_amdgcn_fdot2(u6, ones, b6, false);
            b8 = __builtin_amdgcn_fdot2(u8, ones, b8, false);
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
                const uint32_t x0 = wd ? vw[2 * pp].y : vw[2 * pp].x;
                const uint32_t x1 = wd ? vw[2 * pp + 1].y : vw[2 * pp + 1].x;
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    // bytes hb*2, hb*2+1 of token 2pp (low half) and token 2pp+1 (high half):
                    // channels o+{0,4,8,12} at bits 0,2,4,6 and o+{1,5,9,13} at 8,10,12,14
                    const uint32_t X = __builtin_amdgcn_perm(x1, x0, hb ? 0x07060302u : 0x05040100u);
                    const uint32_t l4 = X << 4, r4 = X >> 4, l8 = X << 8, r8 = X >> 8;
                    const int o = 16 * wd + 2 * hb;
                    acc[o + 0] = fdot2(and_or(l8, kM8, kOne), u8, acc[o + 0]);
                    acc[o + 1] = fdot2(and_or(X, kM8, kOne), u8, acc[o + 1]);
                    acc[o + 4] = fdot2(and_or(l4, kM6, kOne), u6, acc[o + 4]);
                    acc[o + 5] = fdot2(and_or(r4, kM6, kOne), u6, acc[o + 5]);
                    acc[o + 8] = fdot2(and_or(l4, kM8, kOne), u8, acc[o + 8]);
                    acc[o + 9] = fdot2(and_or(r4, kM8, kOne), u8, acc[o + 9]);
                    acc[o + 12] = fdot2(and_or(X, kM6, kOne), u6, acc[o + 12]);
                    acc[o + 13] = fdot2(and_or(r8, kM6, kOne), u6, acc[o + 13]);
                }
            }
        }
        cur = nxt;
    }

    // true partial output of the lane's quarter: sum(w*c) = (acc - bias) / vs, plus p*z
    float o[32];
    {
        const float inv = vs != 0.0f ? 1.0f / vs : 0.0f;
#pragma unroll
        for (int c = 0; c < 32; ++c) o[c] = fmaf(acc[c] - ((c & 4) ? b6 : b8), inv, zacc);
    }

    // fp16 residual, logical tokens [32*wave, 32*wave+32) of the ring, last split only.
    // Lane = 4*tp + qq: tokens 2tp, 2tp+1 of the chunk, channels [32qq, 32qq+32).
    if (split == a.splits - 1 && wave * kG < a.n_res) {
        const int tp = lane >> 2;
        float qv[32];
        load_q32(a.q + qrow * kD + qq * 32, a.sm_log2, qv);
        for (int base = wave * kG; base < a.n_res; base += kWaves * kG) {
            const int i0 = base + 2 * tp, i1 = i0 + 1;
            const bool ok0 = i0 < a.n_res, ok1 = i1 < a.n_res;
            const int s0 = (a.res_head + (ok0 ? i0 : 0)) % a.residual_cap;
            const int s1 = (a.res_head + (ok1 ? i1 : 0)) % a.residual_cap;
            const int64_t r0 = (kvrow * a.residual_cap + s0) * kD + qq * 32;
            const int64_t r1 = (kvrow * a.residual_cap + s1) * kD + qq * 32;
            const uint4* k0 = reinterpret_cast<const uint4*>(a.k_res + r0);
            const uint4* k1 = reinterpret_cast<const uint4*>(a.k_res + r1);
            float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 x0 = k0[i], x1 = k1[i];
                const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w}, w1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int c = 8 * i + 2 * k;
                    d0 = fmaf(qv[c], h2f(w0[k] & 0xffffu), d0);
                    d0 = fmaf(qv[c + 1], h2f(w0[k] >> 16), d0);
                    d1 = fmaf(qv[c], h2f(w1[k] & 0xffffu), d1);
                    d1 = fmaf(qv[c + 1], h2f(w1[k] >> 16), d1);
                }
            }
            d0 = wave_sum_xor(d0, 1, 2);
            d1 = wave_sum_xor(d1, 1, 2);
            const float l0 = ok0 ? d0 : -INFINITY, l1 = ok1 ? d1 : -INFINITY;
            const float m_new = fmaxf(m, wave_max_xor(fmaxf(l0, l1), 4, 32));
            const float alpha = (m == -INFINITY) ? 0.0f : exp2f(m - m_new);
            const float p0 = ok0 ? exp2f(l0 - m_new) : 0.0f;
            const float p1 = ok1 ? exp2f(l1 - m_new) : 0.0f;
            // lsum holds one share per token: the quantized tokens' in the lane that owned
            // them, a residual pair's in the qq = 0 lane of its quad
            lsum = lsum * alpha + (qq == 0 ? p0 + p1 : 0.0f);
            const uint4* v0 = reinterpret_cast<const uint4*>(a.v_res + r0);
            const uint4* v1 = reinterpret_cast<const uint4*>(a.v_res + r1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 x0 = v0[i], x1 = v1[i];
                const uint32_t w0[4] = {x0.x, x0.y, x0.z, x0.w}, w1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int c = 8 * i + 2 * k;
                    o[c] = fmaf(p1, h2f(w1[k] & 0xffffu), fmaf(p0, h2f(w0[k] & 0xffffu), o[c] * alpha));
                    o[c + 1] = fmaf(p1, h2f(w1[k] >> 16), fmaf(p0, h2f(w0[k] >> 16), o[c + 1] * alpha));
                }
            }
            m = m_new;
        }
    }

    // wave result: sum over the 16 lanes that share a channel quarter
    lsum = wave_sum_xor(lsum, 1, 32);
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = wave_sum_xor(o[c], 4, 32);
    if ((lane >> 2) == 0) {
#pragma unroll
        for (int c = 0; c < 32; ++c) sh_o[wave][qq * 32 + c] = o[c];
    }
    if (lane == 0) {
        sh_m[wave] = m;
        sh_l[wave] = lsum;
    }
    __syncthreads();
    float* part = a.ws + ((int64_t)split * a.q_rows + qrow) * kPart;
    if (threadIdx.x < kD) {
        const int j = threadIdx.x;
        float M = sh_m[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh_m[w]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = (sh_m[w] == -INFINITY) ? 0.0f : exp2f(sh_m[w] - M);
            L = fmaf(sh_l[w], sc, L);
            O = fmaf(sh_o[w][j], sc, O);
        }
        store_coherent(&part[j], O);
        if (j == 0) {
            store_coherent(&part[kD], M);
            store_coherent(&part[kD + 1], L);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // those stores have completed
    }
    // The last workgroup of this row to arrive merges every split's partial and writes the
    // output.  The counter add comes after every partial store of this workgroup completed
    // (the wait above, then the barrier), and the merging workgroup issues its coherent loads
    // only after its own add returned the final count, so it reads every partial.
    __syncthreads();
    __shared__ bool sh_last;
    if (threadIdx.x == 0)
        sh_last = __hip_atomic_fetch_add(&a.counters[qrow], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (unsigned)(a.splits - 1);
    __syncthreads();
    if (sh_last) merge_row(a, qrow);
}

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(attn_split_kernel, dim3((unsigned)a.splits, (unsigned)a.q_rows), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace kivi
