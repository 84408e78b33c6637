// kivi_attn_rope.hip -- decode attention over a cache of pre-RoPE keys (gfx950).
//
// Keys are quantized before the rotary position embedding is applied (advised by "Your KV
// cache doesn't have a bit problem...", paragraph 4, and the KVQuant summary on GrooveSquid),
// so attention turns every dequantized key by its position's angles before the dot product.
// Rotary embedding, rotate-half form: channel i < 64 pairs with channel i + 64, pair i turns
// at w_i = base^(-2i/128), a token at position p by p*w_i; positions are sequence indices
// (history token t at t, the i-th oldest residual token at n_quant + i).  With complex pairs
// Q_i = q_i + i*q_{i+64} and K_i = k_i + i*k_{i+64}, the logit is
//     q . rope(k, p) = sum_i Re(conj(Q_i) * K_i * exp(i*p*w_i)).
// The query is used as given (rotated by the caller at its own position); values carry no
// position.
//
// The angle is split as p = t0 + d (t0 the key group's first token, d < G the offset in the
// group).  Once per group a lane forms, for each of its pairs, W = conj(Q)*exp(i*t0*w) and
// the folded products U = W*(z_i + i*z_{i+64}), V = W*s_i, X = i*W*s_{i+64}, so that for a
// token with codes (c, c') W*K = U + V*c + X*c'; per token it then adds
// Re((U + V*c + X*c') * exp(i*d*w)), with exp(i*d*w) from an LDS table.  The turn of the
// group start is reduced modulo 2*pi in binary64 (positions reach 2^17 and more radians),
// its cosine and sine taken in binary32.  The per-pair products make this path bound by the
// vector units rather than by HBM.
//
// Work split: grid (splits, query rows), one query head per workgroup (a GQA group's heads
// each read their KV head); a split owns whole key groups, each of its 4 waves a contiguous
// run of them, 16 tokens per wave-iteration in two passes of 8 (lane 8t + k: token t of the
// pass, pairs [8k, 8k+8)).  P.V follows the code layout of the cache's width: 2-bit value
// tiles (lane: one 8-token row of chunks, 4 channels), 4-bit token rows (lane: 4 tokens, 8
// channels), with the dequantization folded in as (p*s)*c + p*z.
#include <hip/hip_ext.h>

#include "kivi_attn_common.h"

namespace kivi {

constexpr int kRpTok = 16;          // tokens per wave-iteration
constexpr int kRpPairs = kD / 2;    // rotary pairs: channel i with channel i + 64

// cos and sin of theta: reduced to [-pi, pi] in binary64 (2*pi as a two-term sum), then
// sincosf of the binary32 remainder
__device__ __forceinline__ float2 turn(double theta) {
    constexpr double kInv2Pi = 0.15915494309189535;
    constexpr double k2PiHi = 6.283185307179586;        // 2*pi rounded to binary64
    constexpr double k2PiLo = 2.4492935982947064e-16;   // 2*pi - k2PiHi
    const double k = rint(theta * kInv2Pi);
    const double r = fma(-k, k2PiLo, fma(-k, k2PiHi, theta));
    float s, c;
    sincosf((float)r, &s, &c);
    return make_float2(c, s);
}

// Codes of the 8 channels base..base+7 of one token word (see the layouts in the header):
// 2-bit key word (16 channels, channel 16w + 4i + b in byte b at bits 2i): the lane's 8
// channels are the fields i = 2h, 2h+1 (h = lane's half of the word), channel 8h + 4i' + b;
// 4-bit word (8 channels, channel 2b + e in byte b, nibble e).  Returned indexed by channel.
template <int BITS>
__device__ __forceinline__ void codes8(uint32_t w, int h, float (&c)[8]) {
    uint32_t y0, y1;
    if constexpr (BITS == 2) {
        const uint32_t x = w >> (4 * h);
        y0 = x & 0x03030303u;          // channels b      (i' = 0)
        y1 = (x >> 2) & 0x03030303u;   // channels 4 + b  (i' = 1)
    } else {
        y0 = w & 0x0F0F0F0Fu;          // channels 2b
        y1 = (w >> 4) & 0x0F0F0F0Fu;   // channels 2b + 1
    }
    asm volatile("" : "+v"(y0), "+v"(y1));   // one v_cvt_f32_ubyteN per code
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float f0 = (float)((y0 >> (8 * b)) & 0xFFu), f1 = (float)((y1 >> (8 * b)) & 0xFFu);
        if constexpr (BITS == 2) {
            c[b] = f0;
            c[4 + b] = f1;
        } else {
            c[2 * b] = f0;
            c[2 * b + 1] = f1;
        }
    }
}

// Softmax state of query row qrow over the fp16 residual ring, keys turned at positions
// n_quant + i.  Wave w takes the ring's logical tokens w, w + 4, ...; lane m holds pair m
// (channels m, m + 64) for the logit (a wave sum) and the same two channels for P.V.  In a
// fused decode step the last residual token is the new one, read from k_new / v_new.
__device__ void residual_rope_states(const AttnArgs& a, const RowState& rs, int64_t qrow, int64_t kvrow, int wave,
                                     const double* w_pair, float* o_dst, float& mr, float& lr) {
    const int lane = threadIdx.x & 63;
    const float q0 = h2f(a.q[qrow * kD + lane]), q1 = h2f(a.q[qrow * kD + lane + kRpPairs]);
    const double wm = w_pair[lane];
    float o0 = 0.0f, o1 = 0.0f;
    mr = -INFINITY;
    lr = 0.0f;
    for (int i = wave; i < rs.n_res; i += kWaves) {
        const int slot = (rs.res_head + i) % a.residual_cap;
        const bool fresh = a.k_new != nullptr && i == rs.n_res - 1;
        const uint16_t* kr = fresh ? a.k_new + kvrow * kD : a.k_res + (kvrow * a.residual_cap + slot) * kD;
        const uint16_t* vr = fresh ? a.v_new + kvrow * kD : a.v_res + (kvrow * a.residual_cap + slot) * kD;
        const float2 e = turn((double)(rs.n_quant + i) * wm);
        const float wr = fmaf(q0, e.x, q1 * e.y), wi = fmaf(q0, e.y, -q1 * e.x);   // conj(Q) * e
        const float part = fmaf(wr, h2f(kr[lane]), -wi * h2f(kr[lane + kRpPairs]));
        const float lg = wave_sum(part) * a.sm_log2;
        const float mnew = fmaxf(mr, lg);
        const float al = mr == -INFINITY ? 0.0f : exp2f(mr - mnew);
        const float p = exp2f(lg - mnew);
        lr = fmaf(lr, al, p);
        o0 = fmaf(o0, al, p * h2f(vr[lane]));
        o1 = fmaf(o1, al, p * h2f(vr[lane + kRpPairs]));
        mr = mnew;
    }
    o_dst[lane] = o0;
    o_dst[lane + kRpPairs] = o1;
}

template <int BITS, int GS, bool RAGGED>
__global__ __launch_bounds__(kBlock) void attn_rope_kernel(AttnArgs a) {
    constexpr int kIt = GS / kRpTok;   // iterations per key group
    __shared__ double sh_w[kRpPairs];                        // pair frequencies
    __shared__ __align__(16) float2 sh_ed[GS][kRpPairs];     // exp(i*d*w) for offsets d < G
    __shared__ __align__(16) float2 sh_e0[kWaves][kRpPairs]; // exp(i*t0*w) of the wave's group
    __shared__ __align__(16) float sh_p[kWaves][kRpTok];
    __shared__ __align__(16) float sh_ps[kWaves][kD / GS][kRpTok];   // 2-bit: p*s per (value group, token)
    __shared__ __align__(16) float sh_o[1][kSlots][kD];
    __shared__ float sh_m[1][kSlots], sh_l[1][kSlots];

    // (ragged batch: the plan uses sh_o, unused until the end)
    const WorkItem wi = work_item<RAGGED>(a, reinterpret_cast<int32_t*>(&sh_o[0][0][0]));
    if (RAGGED && wi.split < 0) return;   // (ragged batch) past the plan's last item
    const int split = wi.split;
    const int64_t qrow = wi.row;
    // query row b*Hq + h reads kv row b*Hkv + h/ratio = qrow/ratio (Hq = Hkv*ratio)
    const int64_t kvrow = a.ratio == 1 ? qrow : (int64_t)((uint32_t)qrow / (uint32_t)a.ratio);
    if (a.k_new != nullptr && split == 0 && (uint32_t)qrow % (uint32_t)a.ratio == 0) store_new_token(a, kvrow);
    const TagLoads<1> tag_v = partial_tag<1>(a, qrow);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t8 = lane >> 3, k8 = lane & 7;

    const RowState rs = RAGGED ? wi.rs : row_state(a);
    const int n_kg = rs.n_quant / GS;
    const int per_split = (n_kg + rs.splits - 1) / rs.splits;
    const int kg_lo = min(n_kg, split * per_split), kg_hi = min(n_kg, kg_lo + per_split);
    const int cnt = kg_hi - kg_lo;
    const int per_wave = (cnt + kWaves - 1) / kWaves;
    const int kgb = kg_lo + min(cnt, wave * per_wave);
    const int n_groups = kg_lo + min(cnt, (wave + 1) * per_wave) - kgb;
    const int n_it = n_groups * kIt;

    // the lane's query pairs: channels 8k8..8k8+7 and 64+8k8..64+8k8+7
    float qlo[8], qhi[8];
    {
        const uint4 x = *reinterpret_cast<const uint4*>(a.q + qrow * kD + 8 * k8);
        const uint4 y = *reinterpret_cast<const uint4*>(a.q + qrow * kD + kRpPairs + 8 * k8);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qlo[2 * i] = h2f(xs[i] & 0xffffu);
            qlo[2 * i + 1] = h2f(xs[i] >> 16);
            qhi[2 * i] = h2f(ys[i] & 0xffffu);
            qhi[2 * i + 1] = h2f(ys[i] >> 16);
        }
    }

    const int64_t tok0 = kvrow * (int64_t)a.token_cap;
    const uint8_t* kc_row = a.k_codes + tok0 * (BITS == 2 ? kRowBytes : kRowBytes4);
    const uint8_t* vc_row = a.v_codes + tok0 * (BITS == 2 ? kRowBytes : kRowBytes4);
    const uint32_t* kp_row = reinterpret_cast<const uint32_t*>(a.k_sz) + kvrow * (int64_t)(a.token_cap / GS) * kD;
    const uint32_t* vp_row = reinterpret_cast<const uint32_t*>(a.v_sz) + tok0 * (kD / GS);
    const int t_b = kgb * GS;
    auto tok = [&](int it) { return t_b + min(it, n_it - 1) * kRpTok; };   // clamped past the end

    // key codes of the two pass tokens (lo word, hi word each)
    struct KLoad { uint32_t lo[2], hi[2]; };
    auto load_k = [&](KLoad& L, int it) {
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const uint32_t t = (uint32_t)(tok(it) + 8 * ps + t8);
            if constexpr (BITS == 2) {
                // chunk (16w + t%16) of the token's tile, 8-byte half t%32/16: words w, w + 4
                const uint32_t off = (t / kG) * kTileBytes + (16 * (k8 >> 1) + t % 16) * 16 + 8 * ((t % kG) / 16);
                const uint2 x = *reinterpret_cast<const uint2*>(kc_row + off);
                L.lo[ps] = x.x;
                L.hi[ps] = x.y;
            } else {
                const uint8_t* r = kc_row + t * kRowBytes4;
                L.lo[ps] = *reinterpret_cast<const uint32_t*>(r + 4 * k8);
                L.hi[ps] = *reinterpret_cast<const uint32_t*>(r + kRowBytes4 / 2 + 4 * k8);
            }
        }
    };
    // P.V lanes.  2-bit: lane (kk, n, hh) reads bytes 8hh..8hh+7 of chunk (16k + n) of the
    // tile, k = 2*(t0%32/16) + kk: tokens 8kk + 4h + i of the iteration (h = 0..1, i = 0..3)
    // and channels n + 16(4hh + m) (m = 0..3, in word m/2, byte 2h + m%2, bits 2i); with
    // G = 32 channels m = 0, 1 are in value group 2hh and m = 2, 3 in group 2hh + 1.  Each
    // (token, value group) of the iteration has one lane of the softmax octets that loads its
    // (scale, zero) word and forms p*s (into LDS) and p*z (summed in that lane): octet t8,
    // lane k8 < 2*NG takes token t8 + 8*(k8 / NG) and group k8 % NG (NG = 128/G groups).
    // 4-bit: lane (vg, vc) reads tokens 4vg..4vg+3 and channels 8vc..8vc+7 (one group).
    constexpr int kNG = kD / GS;                          // value groups per token
    constexpr int kVGrp = (BITS == 2 && GS == 32) ? 2 : 1;  // value groups per lane and token
    constexpr int kVCh = BITS == 2 ? 4 : 8;               // channels per lane
    const int kk = lane >> 5, vn = (lane >> 1) & 15, hh = lane & 1;
    const int vg = lane >> 4, vc = lane & 15;
    const bool combo = BITS == 2 && k8 < 2 * kNG;
    const int c_tok = t8 + 8 * (min(k8, 2 * kNG - 1) / kNG), c_grp = min(k8, 2 * kNG - 1) % kNG;
    struct VLoad { uint32_t c[4]; uint32_t p[4]; };
    auto load_v = [&](VLoad& L, int it) {
        const uint32_t t0 = (uint32_t)tok(it);
        if constexpr (BITS == 2) {
            const uint32_t off = (t0 / kG) * kTileBytes + ((2 * ((t0 % kG) / 16) + kk) * 16 + vn) * 16 + 8 * hh;
            const uint2 x = *reinterpret_cast<const uint2*>(vc_row + off);
            L.c[0] = x.x;
            L.c[1] = x.y;
            L.p[0] = vp_row[(t0 + c_tok) * kNG + c_grp];   // this lane's (token, group) pair
        } else {
            const uint32_t t = t0 + 4 * vg;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                L.c[u] = *reinterpret_cast<const uint32_t*>(vc_row + (t + u) * kRowBytes4 + 4 * vc);
                L.p[u] = vp_row[(t + u) * (kD / GS) + (8 * vc) / GS];
            }
        }
    };
    // key (scale, zero) words of group gi of the wave, channels 8k8.. and 64+8k8..
    struct PLoad { uint4 lo[2], hi[2]; };
    auto load_kp = [&](PLoad& L, int gi) {
        const uint32_t* g = kp_row + (int64_t)(kgb + min(gi, n_groups - 1)) * kD;
        L.lo[0] = *reinterpret_cast<const uint4*>(g + 8 * k8);
        L.lo[1] = *reinterpret_cast<const uint4*>(g + 8 * k8 + 4);
        L.hi[0] = *reinterpret_cast<const uint4*>(g + kRpPairs + 8 * k8);
        L.hi[1] = *reinterpret_cast<const uint4*>(g + kRpPairs + 8 * k8 + 4);
    };
    auto wave_sync = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    float m = -INFINITY, lsum = 0.0f, o[kVCh], oz = 0.0f;   // oz: 2-bit, the lane's (token, group) p*z; 4-bit, its tokens'
#pragma unroll
    for (int c = 0; c < kVCh; ++c) o[c] = 0.0f;
    float* pw = &sh_p[wave][0];

    KLoad kl;
    VLoad vl;
    PLoad pn;
    if (n_groups > 0) {   // the first iteration's loads, in flight while the turn tables are built
        load_k(kl, 0);
        load_v(vl, 0);
        load_kp(pn, 0);
    }
    // pair frequencies and the in-group turns exp(i*d*w)
    if (threadIdx.x < kRpPairs) sh_w[threadIdx.x] = pow(a.rope_base, -2.0 * (double)threadIdx.x / (double)kD);
    __syncthreads();
    for (int i = threadIdx.x; i < GS * kRpPairs; i += kBlock) sh_ed[i / kRpPairs][i % kRpPairs] = turn((double)(i / kRpPairs) * sh_w[i % kRpPairs]);
    __syncthreads();

    uint32_t tag;
    if (n_groups > 0) {
        tag = settle_tag(tag_v);
        for (int gi = 0; gi < n_groups; ++gi) {
            // ---- turn of the group start for the 64 pairs (lane = pair), through LDS
            sh_e0[wave][lane] = turn((double)((kgb + gi) * GS) * sh_w[lane]);
            wave_sync();
            float ur[8], ui[8], vr[8], vi[8], xr[8], xi[8];
            {
                const uint32_t plo[8] = {pn.lo[0].x, pn.lo[0].y, pn.lo[0].z, pn.lo[0].w,
                                         pn.lo[1].x, pn.lo[1].y, pn.lo[1].z, pn.lo[1].w};
                const uint32_t phi[8] = {pn.hi[0].x, pn.hi[0].y, pn.hi[0].z, pn.hi[0].w,
                                         pn.hi[1].x, pn.hi[1].y, pn.hi[1].z, pn.hi[1].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float2 e = sh_e0[wave][8 * k8 + j];
                    const float wr = fmaf(qlo[j], e.x, qhi[j] * e.y);    // W = conj(Q) * e
                    const float wi = fmaf(qlo[j], e.y, -qhi[j] * e.x);
                    const float slo = h2f(plo[j] & 0xffffu), zlo = h2f(plo[j] >> 16);
                    const float shi = h2f(phi[j] & 0xffffu), zhi = h2f(phi[j] >> 16);
                    ur[j] = fmaf(wr, zlo, -wi * zhi);                    // U = W * (zlo + i*zhi)
                    ui[j] = fmaf(wr, zhi, wi * zlo);
                    vr[j] = wr * slo;                                    // V = W * slo
                    vi[j] = wi * slo;
                    xr[j] = -wi * shi;                                   // X = i * W * shi
                    xi[j] = wr * shi;
                }
            }
            wave_sync();   // every lane has read the turns before the next group's are written
            load_kp(pn, gi + 1);
#pragma unroll 1
            for (int j = 0; j < kIt; ++j) {
                const int it = gi * kIt + j;
                // ---- logits of tokens t8 and 8 + t8 (pass 0, 1), this lane's 8 pairs
                float lg[2];
#pragma unroll
                for (int ps = 0; ps < 2; ++ps) {
                    float c1[8], c2[8];
                    codes8<BITS>(kl.lo[ps], k8 & 1, c1);
                    codes8<BITS>(kl.hi[ps], k8 & 1, c2);
                    const float2* ed = &sh_ed[kRpTok * j + 8 * ps + t8][8 * k8];
                    float acc = 0.0f;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const float2 e = ed[jj];
                        const float kr = fmaf(xr[jj], c2[jj], fmaf(vr[jj], c1[jj], ur[jj]));
                        const float ki = fmaf(xi[jj], c2[jj], fmaf(vi[jj], c1[jj], ui[jj]));
                        acc = fmaf(kr, e.x, fmaf(-ki, e.y, acc));
                    }
                    acc += xor1_f(acc);              // over the token's 8 lanes
                    acc += xor2_f(acc);
                    acc += hmirror_f(acc);
                    lg[ps] = acc * a.sm_log2;
                }
                load_k(kl, it + 1);
                // ---- online softmax over the 16 tokens (values equal inside each octet)
                float mx = fmaxf(lg[0], lg[1]);
                mx = fmaxf(mx, ror8_f(mx));
                mx = fmaxf(mx, xor16_f(mx));
                mx = fmaxf(readlane_f(mx, 0), readlane_f(mx, 32));
                const float mnew = fmaxf(m, mx);
                if (mnew != m) {
                    const float al = m == -INFINITY ? 0.0f : exp2f(m - mnew);
#pragma unroll
                    for (int c = 0; c < kVCh; ++c) o[c] *= al;
                    oz *= al;
                    lsum *= al;
                    m = mnew;
                }
                const float p0 = exp2f(lg[0] - m), p1 = exp2f(lg[1] - m);
                if (k8 == 0) {
                    lsum += p0 + p1;
                    pw[t8] = p0;
                    pw[8 + t8] = p1;
                }
                if constexpr (BITS == 2) {
                    if (combo) {
                        const float pc = c_tok < 8 ? p0 : p1;
                        sh_ps[wave][c_grp][c_tok] = pc * h2f(vl.p[0] & 0xffffu);
                        oz = fmaf(pc, h2f(vl.p[0] >> 16), oz);
                    }
                }
                wave_sync();
                // ---- P.V, dequantization folded: (p*s)*c + p*z
                if constexpr (BITS == 2) {
                    // p*s of the lane's 8 tokens in each of its value groups
                    float ps[kVGrp][8];
#pragma unroll
                    for (int g = 0; g < kVGrp; ++g) {
                        const int grp = GS == 32 ? 2 * hh + g : (GS == 64 ? hh : 0);
                        const float4 a0 = *reinterpret_cast<const float4*>(&sh_ps[wave][grp][8 * kk]);
                        const float4 a1 = *reinterpret_cast<const float4*>(&sh_ps[wave][grp][8 * kk + 4]);
                        ps[g][0] = a0.x; ps[g][1] = a0.y; ps[g][2] = a0.z; ps[g][3] = a0.w;
                        ps[g][4] = a1.x; ps[g][5] = a1.y; ps[g][6] = a1.z; ps[g][7] = a1.w;
                    }
#pragma unroll
                    for (int w2 = 0; w2 < 2; ++w2) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // token field i of word w2: byte 2h + e = channel 2*w2 + e, token 4h + i
                            uint32_t y = (vl.c[w2] >> (2 * i)) & 0x03030303u;
                            asm volatile("" : "+v"(y));   // one v_cvt_f32_ubyteN per code
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                const int mm = 2 * w2 + (b & 1), u = 4 * (b >> 1) + i;
                                const int g = kVGrp == 2 ? w2 : 0;
                                o[mm] = fmaf(ps[g][u], (float)((y >> (8 * b)) & 0xFFu), o[mm]);
                            }
                        }
                    }
                } else {
                    const float4 pa = *reinterpret_cast<const float4*>(pw + 4 * vg);
                    const float pt[4] = {pa.x, pa.y, pa.z, pa.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float s = h2f(vl.p[u] & 0xffffu), z = h2f(vl.p[u] >> 16);
                        const float ps = pt[u] * s;
                        oz = fmaf(pt[u], z, oz);
                        uint32_t lo = vl.c[u] & 0x0F0F0F0Fu, hi = (vl.c[u] >> 4) & 0x0F0F0F0Fu;
                        asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float code = (float)((((c & 1) ? hi : lo) >> (8 * (c >> 1))) & 0xFFu);
                            o[c] = fmaf(ps, code, o[c]);
                        }
                    }
                }
                load_v(vl, it + 1);
                wave_sync();
            }
        }
    } else {
        tag = settle_tag(tag_v);
    }

    // ---- the wave's state: p*z shares added to their channels, lanes of a channel summed
    if constexpr (BITS == 2) {
        // sum of p*z per value group over the wave's tokens, then the lane's groups picked by
        // compare-and-select (an index from hh would put the array in scratch memory)
        float zl[kVGrp];
#pragma unroll
        for (int g2 = 0; g2 < kVGrp; ++g2) zl[g2] = 0.0f;
#pragma unroll
        for (int g = 0; g < kNG; ++g) {
            const float t = wave_sum(combo && c_grp == g ? oz : 0.0f);
#pragma unroll
            for (int g2 = 0; g2 < kVGrp; ++g2) {
                const int want = GS == 32 ? 2 * hh + g2 : (GS == 64 ? hh : 0);
                zl[g2] = g == want ? t : zl[g2];
            }
        }
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
            float x = o[mm];
            x += __shfl_xor(x, 32, 64);                  // the two 8-token rows (kk)
            if (kk == 0) sh_o[0][wave][vn + 16 * (4 * hh + mm)] = x + zl[kVGrp == 2 ? (mm >> 1) : 0];
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float x = o[c] + oz;
            x += xor16_f(x);
            x += __shfl_xor(x, 32, 64);                  // the four token quads (vg)
            if (lane < 16) sh_o[0][wave][8 * vc + c] = x;
        }
    }
    const float l = wave_sum(lsum);
    if (lane == 0) {
        sh_m[0][wave] = n_groups > 0 ? m : -INFINITY;
        sh_l[0][wave] = l;
    }
    // ---- fp16 residual (split rs.res_split), keys turned at n_quant + i
    float mr = -INFINITY, lr = 0.0f;
    if (split == rs.res_split) residual_rope_states(a, rs, qrow, kvrow, wave, sh_w, &sh_o[0][kWaves + wave][0], mr, lr);
    if (lane == 0) {
        sh_m[0][kWaves + wave] = mr;
        sh_l[0][kWaves + wave] = lr;
    }
    __syncthreads();
    finish_block<1>(a, rs.splits, split, qrow, tag, sh_o, sh_m, sh_l);
}

hipError_t launch_decode_attn_rope(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = attn_grid(a, a.q_rows);
#define KIVI_ROPE(BITSv, RAGGEDv)                                                                                  \
    KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_rope_kernel<BITSv, GS, RAGGEDv>), grid, dim3(kBlock), 0, s, t0, t1, \
                                                 0, a))
    const bool ragged = a.seq_state != nullptr;
    if (a.bits == 4) {
        if (ragged) KIVI_ROPE(4, true) else KIVI_ROPE(4, false)
    } else {
        if (ragged) KIVI_ROPE(2, true) else KIVI_ROPE(2, false)
    }
#undef KIVI_ROPE
    return hipGetLastError();
}

}  // namespace kivi
