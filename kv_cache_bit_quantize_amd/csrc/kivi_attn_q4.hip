// kivi_attn_q4.hip -- fused decode attention over a cache of 4-bit codes (gfx950).
//
// The 4-bit member of the quantizer family (sixteen levels; the KIVI summary page names the
// 2-bit one, KIVI-2, and its ablation varies the scheme's parameters): the same call shape,
// query grouping, split-K, fp16 residual and log-sum-exp merge as the 2-bit kernels, with
// the dequantization folded into both products:
//  * keys, per group: q.(z + c*s) = q.z + (q*s).c.  Once per group the wave forms q*s for
//    the 128 channels in fp32 (a product of two fp16 values, exact), turns it into 30-bit
//    fixed point with one exponent per head and stores its four signed byte digits as digit
//    planes in LDS.  The (q*s).c products then run on the matrix cores,
//    v_mfma_i32_16x16x64_i8, exactly: B is the 16 tokens' codes (a lane's 8 bytes of one
//    token row, low and high nibbles masked into bytes, which sets the channel order of the
//    planes), A the digit planes (rows 4r..4r+3 head r's digits, other rows zero), so lane
//    16r + n ends with head r's four digit sums of token n.  q.z is one wave sum per group;
//  * values, per token: p*(z + c*s) = (p*s)*c + p*z on the vector units (the token-major
//    rows do not give the value matrix operand, which needs 8 tokens of one channel per
//    lane): one v_dot2_f32_f16 takes two tokens of one channel, their fp16 weights p*s*vs
//    (vs a power of two shared by the wave, keeping them below 2^14) against their codes,
//    moved by one byte permute into the low bits of each half, where they read as the fp16
//    subnormals c*2^-24 (a high nibble as 16c*2^-24, scaled back at the end): no conversion.
//    The p*z part is summed per lane and added to its channels at the end.
//
// Work split: grid (splits, kv heads x query chunks of NQ heads); a split owns whole key
// groups, each of its 4 waves a contiguous run of them, 16 tokens per wave-iteration:
//  * logits as above, online softmax per query head (log2 domain) over DPP row r, the
//    probabilities into LDS;
//  * P.V: lane 16g + c holds tokens g, g+4, g+8, g+12 and channels [8c, 8c+8) (4 bytes of
//    codes and the token's (scale, zero) word of those channels).
// Code loads are issued one iteration ahead, the next group's (scale, zero) words one group
// ahead, all unconditionally (clamped past the end).  Each code load instruction reads whole
// rows (a lane 16 bytes of a token's key codes, four lanes the row; a value load four
// consecutive rows), so the codes and key pairs stream with non-temporal loads: 107.5-108 us
// at the 131,072-token context against 121.3-121.7 us with plain loads of half rows (same GPU;
// the hint on loads that split rows between instructions had been 9% slower).
#include <hip/hip_ext.h>

#include "kivi_attn_common.h"

namespace kivi {

constexpr int kQ4Tok = 16;   // tokens per wave-iteration

template <int NQ, int GS, bool RAGGED>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void attn_q4_kernel(AttnArgs a) {
    constexpr int kIt = GS / kQ4Tok;   // iterations per key group
    __shared__ __align__(16) float sh_p[kWaves][NQ][kQ4Tok];
    // digit planes of q*s for the wave's current key group: [head][digit][16-channel block w]
    // [position p], position p holding channel 16w + (p & 8) + 2(p & 3) + ((p >> 2) & 1), the
    // order in which a masked token-major code word enters the matrix instruction
    __shared__ __align__(16) uint8_t sh_dg[kWaves][NQ][4][8][16];
    __shared__ __align__(16) uint8_t sh_zero[16];           // the A operand of unused rows
    __shared__ __align__(16) float sh_o[NQ][kSlots][kD];
    __shared__ float sh_m[NQ][kSlots], sh_l[NQ][kSlots];

    // (ragged batch: the plan uses sh_o, unused until the end)
    const WorkItem wi = work_item<RAGGED>(a, reinterpret_cast<int32_t*>(&sh_o[0][0][0]));
    if (RAGGED && wi.split < 0) return;   // (ragged batch) past the plan's last item
    const int split = wi.split;
    const int64_t grow = wi.row;                      // (batch, kv head, query chunk)
    const int chunks = a.ratio / NQ;
    // grow = kvrow*chunks + chunk and Hq = Hkv*ratio = Hkv*chunks*NQ, so the first query row is
    // kvrow*ratio + chunk*NQ = grow*NQ: one 32-bit division (none when a kv head's query group
    // is one workgroup) before the first loads
    const int64_t kvrow = chunks == 1 ? grow : (int64_t)((uint32_t)grow / (uint32_t)chunks);
    const int chunk = (int)(grow - kvrow * chunks);
    const int64_t qrow0 = grow * NQ;
    if (a.k_new != nullptr && split == 0 && chunk == 0) store_new_token(a, kvrow);
    const TagLoads<NQ> tag_v = partial_tag<NQ>(a, qrow0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int mrow = lane & 15, kb = lane >> 4;   // matrix roles: token / A row, K block
    const int vg = lane >> 4, vc = lane & 15;

    const RowState rs = RAGGED ? wi.rs : row_state(a);
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
        uint2 kc[2];      // key codes of token mrow, channels 16(2kb + h)..+15 (h = 0, 1)
        uint32_t v[4];    // value codes of tokens vg+4u, channels 8vc..8vc+7
        uint32_t vp[4];   // (scale, zero) word of those tokens and channels
    };
    auto tok = [&](int it) { return t_b + min(it, n_it - 1) * kQ4Tok; };   // clamped past the end
    // byte offsets inside a row fit 32 bits (token_cap <= 2^26 for 4-bit caches), so the
    // loads take the row pointer as their scalar base and per-token steps as immediates
    auto load_k = [&](Loads& L, int it) {
        const uint8_t* r = kc_row + (uint32_t)(tok(it) + mrow) * kRowBytes4 + 16 * kb;
        const uint4 x = stream_load16(r);
        L.kc[0] = make_uint2(x.x, x.y);
        L.kc[1] = make_uint2(x.z, x.w);
    };
    auto load_v = [&](Loads& L, int it) {
        const uint32_t t = (uint32_t)(tok(it) + vg);
        const uint8_t* cp = vc_row + (t * kRowBytes4 + 4 * vc);
        const uint32_t* pp = vp_row + (t * (kD / GS) + (8 * vc) / GS);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            L.v[u] = stream_load4(cp + 4 * u * kRowBytes4);
            L.vp[u] = pp[4 * u * (kD / GS)];
        }
    };
    // (scale, zero) words of key group gi of the wave, channels 2*lane and 2*lane+1
    auto load_kp = [&](int gi) {
        return stream_load8(kp_row + (int64_t)(kgb + min(gi, n_groups - 1)) * kD + 2 * lane);
    };

    float m[NQ], lsum[NQ], o[NQ][8], oz[NQ];   // oz: sum of p*z of the lane's tokens and channel group
    float vs = 0.0f;                             // the value weights' power of two
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

    if (lane < 16) sh_zero[lane] = 0;
    uint32_t tag;
    if (n_groups > 0) {
        Loads cur;
        load_k(cur, 0);
        load_v(cur, 0);
        uint2 kpn = load_kp(0);
        tag = settle_tag(tag_v);
        for (int gi = 0; gi < n_groups; ++gi) {
            set_priority_for(n_groups - gi);   // (as in the query-group kernel: most work left issues first)
            // this group's q*s (channels 2*lane, 2*lane+1; a product of two fp16 values, exact
            // in fp32) as 30-bit fixed point with one exponent per head (|q*s| * 2^sh < 2^29,
            // truncated: off by less than 2^-29 of the group's largest term), split into four
            // signed base-256 digits and stored into the digit planes; q.z over the wave
            float qz[NQ], unit[NQ];   // unit: 2^-sh, the weight of digit 0
            {
                const float s0 = h2f(kpn.x & 0xffffu), z0 = h2f(kpn.x >> 16);
                const float s1 = h2f(kpn.y & 0xffffu), z1 = h2f(kpn.y >> 16);
                const int w = lane >> 3, q = 2 * (lane & 7);           // channel 2*lane = 16w + q
                const int p0 = (q & 8) + ((q & 6) >> 1), p1 = p0 + 4;  // positions of channels q, q + 1
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const float x0 = q0[r] * s0, x1 = q1[r] * s1;
                    float mx = half_max_nonneg(fmaxf(fabsf(x0), fabsf(x1)));
                    mx = fmax_ieee(readlane_f(mx, 0), readlane_f(mx, 32));
                    const int sh = min(29 - __builtin_amdgcn_frexp_expf(mx), 100);
                    const float fs = __builtin_ldexpf(1.0f, sh);
                    unit[r] = __builtin_ldexpf(1.0f, -sh);
                    const uint32_t d0 = ((uint32_t)(int)(x0 * fs) + 0x80808080u) ^ 0x80808080u;
                    const uint32_t d1 = ((uint32_t)(int)(x1 * fs) + 0x80808080u) ^ 0x80808080u;
#pragma unroll
                    for (int dd = 0; dd < 4; ++dd) {
                        sh_dg[wave][r][dd][w][p0] = (uint8_t)(d0 >> (8 * dd));
                        sh_dg[wave][r][dd][w][p1] = (uint8_t)(d1 >> (8 * dd));
                    }
                    qz[r] = wave_sum(fmaf(q0[r], z0, q1[r] * z1));
                }
            }
            wave_sync();
            kpn = load_kp(gi + 1);
#pragma unroll 1
            for (int j = 0; j < kIt; ++j) {
                const int it = gi * kIt + j;
                // ---- logits on the matrix cores: B = the 16 tokens' codes (a lane's 8 bytes of
                // token mrow, low and high nibbles masked into bytes), A = the digit planes (rows
                // 4r..4r+3: head r's digits 0..3, other rows zero); K = 64 channels per
                // instruction.  Lane 16r + n ends with the four digit sums of head r, token n.
                v4i cacc = {0, 0, 0, 0};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t d0 = cur.kc[h].x, d1 = cur.kc[h].y;
                    const v4i bop = {(int)(d0 & 0x0F0F0F0Fu), (int)((d0 >> 4) & 0x0F0F0F0Fu), (int)(d1 & 0x0F0F0F0Fu),
                                     (int)((d1 >> 4) & 0x0F0F0F0Fu)};
                    const uint8_t* ap = mrow < 4 * NQ ? &sh_dg[wave][mrow >> 2][mrow & 3][2 * kb + h][0] : sh_zero;
                    cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const v4i*>(ap), bop, cacc, 0, 0, 0);
                }
                load_k(cur, it + 1);
                const int hr = lane >> 4;   // the head whose digit sums this lane holds
                float lg = -INFINITY;
                if (hr < NQ) {
                    // digit sums: |S| < 128 * 128 * 15, the total one binary32 rounding
                    const int hw = cacc[3] * 256 + cacc[2], lw = cacc[1] * 256 + cacc[0];
                    const float tot = fmaf((float)hw, 65536.0f, (float)lw);
                    float u = unit[0], z = qz[0];
#pragma unroll
                    for (int r = 1; r < NQ; ++r)
                        if (hr == r) {
                            u = unit[r];
                            z = qz[r];
                        }
                    lg = fmaf(tot, u, z) * a.sm_log2;
                }
                // ---- online softmax per query head over the 16 tokens (head r: DPP row r)
                const float rmx = row_max(lg);
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const float mnew = fmax_ieee(m[r], readlane_f(rmx, 16 * r));
                    if (mnew != m[r]) {
                        const float al = m[r] == -INFINITY ? 0.0f : exp2_fast(m[r] - mnew);
#pragma unroll
                        for (int c = 0; c < 8; ++c) o[r][c] *= al;
                        oz[r] *= al;
                        lsum[r] *= al;
                        m[r] = mnew;
                    }
                    if (hr == r) {
                        const float p = exp2_fast(lg - m[r]);
                        lsum[r] += p;   // the lanes of head r's row, one token each
                        pw[r * kQ4Tok + 4 * (mrow & 3) + (mrow >> 2)] = p;   // token mrow at 4 (mrow % 4) + mrow / 4
                    }
                }
                wave_sync();
                // ---- P.V: tokens vg + 4u (u = 0..3; their weights sit at 4vg + u), channels 8vc..8vc+7
                float pv[NQ][4];
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const float4 x = *reinterpret_cast<const float4*>(pw + r * kQ4Tok + 4 * vg);
                    pv[r][0] = x.x;
                    pv[r][1] = x.y;
                    pv[r][2] = x.z;
                    pv[r][3] = x.w;
                }
                float smax = 0.0f;
#pragma unroll
                for (int u = 0; u < 4; ++u) smax = fmaxf(smax, h2f(cur.vp[u] & 0xffffu));
                if (__builtin_amdgcn_ballot_w64(smax * vs > 16384.0f || (vs == 0.0f && smax > 0.0f))) {
                    const float gm = wave_max_xor(smax, 1, 32);
                    const float nvs = __builtin_ldexpf(1.0f, 14 - __builtin_amdgcn_frexp_expf(gm));
                    if (vs != 0.0f && nvs < vs) {
                        const float rs_ = nvs / vs;
#pragma unroll
                        for (int r = 0; r < NQ; ++r)
#pragma unroll
                            for (int c = 0; c < 8; ++c) o[r][c] *= rs_;
                    }
                    if (vs == 0.0f || nvs < vs) vs = nvs;
                }
                uint32_t cl[2][4], ch[2][4];   // [token pair (u = 0,1 / 2,3)][byte]: channels 8vc + 2b, 8vc + 2b + 1
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // byte b of the pair's first word in byte 0, of its second in byte 2
                        const uint32_t x = __builtin_amdgcn_perm(cur.v[2 * j + 1], cur.v[2 * j], 0x0C000C00u | ((4u + b) << 16) | b);
                        cl[j][b] = x & 0x000F000Fu;
                        ch[j][b] = x & 0x00F000F0u;
                    }
                float sv[4], zv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sv[u] = h2f(cur.vp[u] & 0xffffu) * vs;
                    zv[u] = h2f(cur.vp[u] >> 16);
                }
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    oz[r] = fmaf(pv[r][0], zv[0], fmaf(pv[r][1], zv[1], fmaf(pv[r][2], zv[2], fmaf(pv[r][3], zv[3], oz[r]))));
                    const h2v w0 = {(_Float16)(pv[r][0] * sv[0]), (_Float16)(pv[r][1] * sv[1])};
                    const h2v w1 = {(_Float16)(pv[r][2] * sv[2]), (_Float16)(pv[r][3] * sv[3])};
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        o[r][2 * b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, cl[0][b]), w0, o[r][2 * b], false);
                        o[r][2 * b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, cl[1][b]), w1, o[r][2 * b], false);
                        o[r][2 * b + 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, ch[0][b]), w0, o[r][2 * b + 1], false);
                        o[r][2 * b + 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, ch[1][b]), w1, o[r][2 * b + 1], false);
                    }
                }
                load_v(cur, it + 1);
                wave_sync();
            }
        }
    } else {
        tag = settle_tag(tag_v);
    }

    // ---- the wave's state per query head: o = P.V * 2^24 / vs (odd channels 2^20 / vs) plus
    // the p*z shares, the four token groups' shares summed (lanes c, c+16, c+32, c+48), l summed
    // over the wave (each token counted by its 4 lanes)
    const float inv = vs != 0.0f ? 16777216.0f / vs : 0.0f;
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            // the lane's p*z share belongs to each of its channels
            const float oc = fmaf(o[r][c], (c & 1) ? inv * 0.0625f : inv, oz[r]);
            float x = oc + xor16_f(oc);
            x += __shfl_xor(x, 32, 64);
            o[r][c] = x;
        }
        const float l = wave_sum(lsum[r]);
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
    __builtin_amdgcn_s_setprio(0);
    if (split == rs.res_split) {
        __builtin_amdgcn_s_setprio(2);   // the residual is work the other splits do not have
        residual_states<NQ>(a, rs, qrow0, kvrow, wave, &sh_o[0][kWaves + wave][0], kSlots * kD, mr, lr);
        __builtin_amdgcn_s_setprio(0);
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
    finish_block<NQ>(a, rs.splits, split, qrow0, tag, sh_o, sh_m, sh_l);
}

hipError_t launch_decode_attn_q4(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = attn_grid(a, a.block_rows);
#define KIVI_Q4_NQ(NQv)                                                                                         \
    if (a.seq_state != nullptr)                                                                                 \
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_q4_kernel<NQv, GS, true>), grid, dim3(kBlock), 0, s, t0, \
                                                     t1, 0, a))                                                 \
    else                                                                                                        \
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_q4_kernel<NQv, GS, false>), grid, dim3(kBlock), 0, s, t0, \
                                                     t1, 0, a))
    switch (a.nq) {   // the host takes one, two or four query heads per workgroup for 4-bit caches
        case 1: KIVI_Q4_NQ(1) break;
        case 2: KIVI_Q4_NQ(2) break;
        case 4: KIVI_Q4_NQ(4) break;
        default: return hipErrorInvalidValue;
    }
#undef KIVI_Q4_NQ
    return hipGetLastError();
}

}  // namespace kivi
