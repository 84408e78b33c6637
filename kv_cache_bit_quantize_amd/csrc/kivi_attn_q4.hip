// kivi_attn_q4.hip -- fused decode attention over a cache of 4-bit codes (gfx950).
//
// The 4-bit member of the quantizer family (sixteen levels; the KIVI summary page names the
// 2-bit one, KIVI-2, and its ablation varies the scheme's parameters): the same call shape,
// query grouping, split-K, fp16 residual and log-sum-exp merge as the 2-bit kernels.  A
// 4-bit cache holds twice the code bytes per token, so the contraction runs on the vector
// units, with the dequantization folded into both products:
//  * keys, per group: q.(z + c*s) = q.z + (q*s).c.  Once per group the wave forms q*s for
//    the 128 channels in fp32 (a product of two fp16 values, exact) into LDS and q.z as one
//    wave sum; per token each code then costs one byte-to-float conversion and one fma;
//  * values, per token: p*(z + c*s) = (p*s)*c + p*z, the p*z part summed per lane and
//    added to its channels at the end.
//
// Work split: grid (splits, kv heads x query chunks of NQ heads); a split owns whole key
// groups, each of its 4 waves a contiguous run of them, 16 tokens per wave-iteration:
//  * logits: lane 4t + c holds token t and channels [32c, 32c+32) (16 bytes of codes) and
//    keeps the group's q*s of those channels in registers;
//  * online softmax per query head (log2 domain), the probabilities into LDS;
//  * P.V: lane 16g + c holds tokens 4g..4g+3 and channels [8c, 8c+8) (4 bytes of codes and
//    the token's (scale, zero) word of those channels).
// Code loads are issued one iteration ahead, the next group's (scale, zero) words one group
// ahead, all unconditionally (clamped past the end).
#include <hip/hip_ext.h>

#include "kivi_attn_common.h"

namespace kivi {

constexpr int kQ4Tok = 16;   // tokens per wave-iteration

template <int NQ, int GS>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void attn_q4_kernel(AttnArgs a) {
    constexpr int kIt = GS / kQ4Tok;   // iterations per key group
    __shared__ __align__(16) float sh_p[kWaves][NQ][kQ4Tok];
    __shared__ __align__(16) float sh_qs[kWaves][NQ][kD];   // q*s of the wave's current key group
    __shared__ __align__(16) float sh_o[NQ][kSlots][kD];
    __shared__ float sh_m[NQ][kSlots], sh_l[NQ][kSlots];

    const int split = grid_split(a);
    const int64_t grow = grid_row(a);                 // (batch, kv head, query chunk)
    const int chunks = a.ratio / NQ;
    const int64_t kvrow = grow / chunks;
    const int chunk = (int)(grow % chunks);
    const int64_t qrow0 = (kvrow / a.kv_heads) * a.q_heads + (kvrow % a.kv_heads) * a.ratio + chunk * NQ;
    if (a.k_new != nullptr && split == 0 && chunk == 0) store_new_token(a, kvrow);
    const uint32_t tag_v = partial_tag(a, grow);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kt = lane >> 2, kq = lane & 3;
    const int vg = lane >> 4, vc = lane & 15;

    const RowState rs = row_state(a, kvrow, split);
    if (split >= rs.splits) return;   // (ragged batch) this row uses fewer splits
    // whole key groups: this split's share, then this wave's
    const int n_kg = rs.n_quant / GS;
    const int per_split = (n_kg + rs.splits - 1) / rs.splits;
    const int kg_lo = min(n_kg, split * per_split), kg_hi = min(n_kg, kg_lo + per_split);
    const int cnt = kg_hi - kg_lo;
    const int per_wave = (cnt + kWaves - 1) / kWaves;
    const int kgb = kg_lo + min(cnt, wave * per_wave);
    const int n_groups = kg_lo + min(cnt, (wave + 1) * per_wave) - kgb;
    const int n_it = n_groups * kIt;

    // query channels 2*lane and 2*lane+1 of the NQ heads (the channels whose key pairs this
    // lane loads)
    float q0[NQ], q1[NQ];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(a.q + (qrow0 + r) * kD + 2 * lane);
        q0[r] = h2f(x & 0xffffu);
        q1[r] = h2f(x >> 16);
    }

    const int64_t tok0 = kvrow * (int64_t)a.token_cap;
    const uint8_t* kc_row = a.k_codes + tok0 * kRowBytes4;
    const uint8_t* vc_row = a.v_codes + tok0 * kRowBytes4;
    const uint32_t* kp_row = reinterpret_cast<const uint32_t*>(a.k_sz) + kvrow * (int64_t)(a.token_cap / GS) * kD;
    const uint32_t* vp_row = reinterpret_cast<const uint32_t*>(a.v_sz) + tok0 * (kD / GS);
    const int t_b = kgb * GS;
    struct Loads {
        uint4 k;          // key codes of token kt, channels 32kq..32kq+31
        uint32_t v[4];    // value codes of tokens 4vg+u, channels 8vc..8vc+7
        uint32_t vp[4];   // (scale, zero) word of those tokens and channels
    };
    auto tok = [&](int it) { return t_b + min(it, n_it - 1) * kQ4Tok; };   // clamped past the end
    // byte offsets inside a row fit 32 bits (token_cap <= 2^26 for 4-bit caches), so the
    // loads take the row pointer as their scalar base and per-token steps as immediates
    auto load_k = [&](Loads& L, int it) {
        const uint32_t off = (uint32_t)(tok(it) + kt) * kRowBytes4 + 16 * kq;
        L.k = *reinterpret_cast<const uint4*>(kc_row + off);
    };
    auto load_v = [&](Loads& L, int it) {
        const uint32_t t = (uint32_t)(tok(it) + 4 * vg);
        const uint8_t* cp = vc_row + (t * kRowBytes4 + 4 * vc);
        const uint32_t* pp = vp_row + (t * (kD / GS) + (8 * vc) / GS);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            L.v[u] = *reinterpret_cast<const uint32_t*>(cp + u * kRowBytes4);
            L.vp[u] = pp[u * (kD / GS)];
        }
    };
    // (scale, zero) words of key group gi of the wave, channels 2*lane and 2*lane+1
    auto load_kp = [&](int gi) {
        return *reinterpret_cast<const uint2*>(kp_row + (int64_t)(kgb + min(gi, n_groups - 1)) * kD + 2 * lane);
    };

    float m[NQ], lsum[NQ], o[NQ][8], oz[NQ];   // oz: sum of p*z of the lane's tokens and channel group
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        m[r] = -INFINITY;
        lsum[r] = 0.0f;
        oz[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[r][c] = 0.0f;
    }
    float* pw = &sh_p[wave][0][0];
    auto wave_sync = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    uint32_t tag;
    if (n_groups > 0) {
        Loads cur;
        load_k(cur, 0);
        load_v(cur, 0);
        uint2 kpn = load_kp(0);
        tag = settle_tag(tag_v);
        for (int gi = 0; gi < n_groups; ++gi) {
            // this group's q*s into LDS (channels 2*lane, 2*lane+1) and q.z over the wave
            float qz[NQ];
            {
                const float s0 = h2f(kpn.x & 0xffffu), z0 = h2f(kpn.x >> 16);
                const float s1 = h2f(kpn.y & 0xffffu), z1 = h2f(kpn.y >> 16);
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    *reinterpret_cast<float2*>(&sh_qs[wave][r][2 * lane]) = make_float2(q0[r] * s0, q1[r] * s1);
                    qz[r] = wave_sum(fmaf(q0[r], z0, q1[r] * z1));
                }
            }
            wave_sync();
            float qs[NQ][32];   // q*s of channels 32kq..32kq+31
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 x = *reinterpret_cast<const float4*>(&sh_qs[wave][r][32 * kq + 4 * i]);
                    qs[r][4 * i] = x.x;
                    qs[r][4 * i + 1] = x.y;
                    qs[r][4 * i + 2] = x.z;
                    qs[r][4 * i + 3] = x.w;
                }
            }
            wave_sync();   // every lane has read the group's q*s before the next group's are written
            kpn = load_kp(gi + 1);
#pragma unroll 1
            for (int j = 0; j < kIt; ++j) {
                const int it = gi * kIt + j;
                // ---- logits: 32 channels of token kt for every query head (q.z once per token)
                const uint32_t cw[4] = {cur.k.x, cur.k.y, cur.k.z, cur.k.w};
                float d[NQ];
#pragma unroll
                for (int r = 0; r < NQ; ++r) d[r] = kq == 0 ? qz[r] : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // word i: channels 8i..8i+7 of the quarter, channel 8i + c at bit 4c; the
                    // even channels' codes as the bytes of lo, the odd ones' of hi
                    uint32_t lo = cw[i] & 0x0F0F0F0Fu, hi = (cw[i] >> 4) & 0x0F0F0F0Fu;
                    // opaque to the optimizer, so each code converts with one v_cvt_f32_ubyteN
                    asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float code = (float)((((c & 1) ? hi : lo) >> (8 * (c >> 1))) & 0xFFu);
#pragma unroll
                        for (int r = 0; r < NQ; ++r) d[r] = fmaf(qs[r][8 * i + c], code, d[r]);
                    }
                }
                load_k(cur, it + 1);
                // ---- online softmax per query head over the 16 tokens
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const float lg = quad_sum(d[r]) * a.sm_log2;
                    const float mnew = fmaxf(m[r], wave_max_quads(lg));
                    if (mnew != m[r]) {
                        const float al = m[r] == -INFINITY ? 0.0f : exp2f(m[r] - mnew);
#pragma unroll
                        for (int c = 0; c < 8; ++c) o[r][c] *= al;
                        oz[r] *= al;
                        lsum[r] *= al;
                        m[r] = mnew;
                    }
                    const float p = exp2f(lg - m[r]);
                    lsum[r] += p;   // every lane of the token's quad adds it: divided by 4 below
                    if (kq == 0) pw[r * kQ4Tok + kt] = p;
                }
                wave_sync();
                // ---- P.V: tokens 4vg..4vg+3, channels 8vc..8vc+7
                float pv[NQ][4];
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const float4 x = *reinterpret_cast<const float4*>(pw + r * kQ4Tok + 4 * vg);
                    pv[r][0] = x.x;
                    pv[r][1] = x.y;
                    pv[r][2] = x.z;
                    pv[r][3] = x.w;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float s = h2f(cur.vp[u] & 0xffffu), z = h2f(cur.vp[u] >> 16);
                    uint32_t lo = cur.v[u] & 0x0F0F0F0Fu, hi = (cur.v[u] >> 4) & 0x0F0F0F0Fu;
                    asm volatile("" : "+v"(lo), "+v"(hi));
                    float ps[NQ];
#pragma unroll
                    for (int r = 0; r < NQ; ++r) {
                        const float pt = pv[r][u];
                        ps[r] = pt * s;
                        oz[r] = fmaf(pt, z, oz[r]);
                    }
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float code = (float)((((c & 1) ? hi : lo) >> (8 * (c >> 1))) & 0xFFu);
#pragma unroll
                        for (int r = 0; r < NQ; ++r) o[r][c] = fmaf(ps[r], code, o[r][c]);
                    }
                }
                load_v(cur, it + 1);
                wave_sync();
            }
        }
    } else {
        tag = settle_tag(tag_v);
    }

    // ---- the wave's state per query head: the four token groups' shares of o summed
    // (lanes c, c+16, c+32, c+48), l summed over the wave (each token counted by its 4 lanes)
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float oc = o[r][c] + oz[r];   // the lane's p*z share belongs to each of its channels
            float x = oc + xor16_f(oc);
            x += __shfl_xor(x, 32, 64);
            o[r][c] = x;
        }
        const float l = wave_sum(lsum[r]) * 0.25f;
        if (lane < 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) sh_o[r][wave][8 * vc + c] = o[r][c];
        }
        if (lane == 0) {
            sh_m[r][wave] = n_groups > 0 ? m[r] : -INFINITY;
            sh_l[r][wave] = l;
        }
    }
    // ---- fp16 residual (split rs.res_split), as separate states
    float mr[NQ], lr[NQ];
    if (split == rs.res_split) {
        residual_states<NQ>(a, rs, qrow0, kvrow, wave, &sh_o[0][kWaves + wave][0], kSlots * kD, mr, lr);
    } else {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            mr[r] = -INFINITY;
            lr[r] = 0.0f;
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            sh_m[r][kWaves + wave] = mr[r];
            sh_l[r][kWaves + wave] = lr[r];
        }
    }
    __syncthreads();
    finish_block<NQ>(a, rs.splits, split, qrow0, grow, tag, sh_o, sh_m, sh_l);
}

hipError_t launch_decode_attn_q4(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = attn_grid(a, a.block_rows);
#define KIVI_Q4_NQ(NQv)                                                                                         \
    KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_q4_kernel<NQv, GS>), grid, dim3(kBlock), 0, s, t0, t1, 0, a))
    switch (a.nq) {   // the host takes at most two query heads per workgroup for 4-bit caches
        case 1: KIVI_Q4_NQ(1) break;
        case 2: KIVI_Q4_NQ(2) break;
        default: return hipErrorInvalidValue;
    }
#undef KIVI_Q4_NQ
    return hipGetLastError();
}

}  // namespace kivi
