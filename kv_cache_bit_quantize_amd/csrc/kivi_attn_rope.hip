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
// Re((U + V*c + X*c') * exp(i*d*w)), with exp(i*d*w) from an LDS table.  Where the turn of
// a group start is taken from its angle, the angle is reduced modulo 2*pi in binary64
// (positions reach 2^17 and more radians) and its cosine and sine taken in binary32; a wave's
// next groups turn by products with exp(i*G*w) (GroupTurn).  The per-pair products make this
// path bound by the vector units rather than by HBM.
//
// Work split: grid (splits, query rows), one query head per workgroup (GQA ratios divisible by
// neither 2 nor 3; a GQA group's heads each read their KV head; the query-group
// form further down takes the rest); a split owns whole key groups, each of its 4 waves a contiguous
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

// The turns exp(i*t0*w) of a wave's consecutive key groups (t0 = G*g): the first from the
// angle (turn), each next one as the product with exp(i*G*w), and again from the angle every
// kReanchor groups.  A product in binary32 moves the phase and the length by a few units of
// 2^-24, so the turn drifts by under 1e-5 between anchors, far below the logits' tolerance,
// and a group's turn costs four operations instead of a reduction and a sincos.
constexpr int kReanchor = 16;
struct GroupTurn {
    float2 e, step;
    double w;
    __device__ __forceinline__ void init(double w_pair, int gs) {
        w = w_pair;
        step = turn((double)gs * w_pair);
    }
    // the turn of group g, the wave's gi-th (groups gi - 1 and gi consecutive for gi > 0)
    __device__ __forceinline__ float2 next(int gi, int64_t t0) {
        if (gi % kReanchor == 0) e = turn((double)t0 * w);
        else e = make_float2(fmaf(e.x, step.x, -e.y * step.y), fmaf(e.x, step.y, e.y * step.x));
        return e;
    }
};

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
    // the key and value channels lane, lane + 64 of residual token i, loaded a token ahead
    struct RLoad { uint16_t k0, k1, v0, v1; };
    auto load = [&](RLoad& L, int i) {
        const int slot = (rs.res_head + i) % a.residual_cap;
        const bool fresh = a.k_new != nullptr && i == rs.n_res - 1;
        const uint16_t* kr = fresh ? a.k_new + kvrow * kD : a.k_res + (kvrow * a.residual_cap + slot) * kD;
        const uint16_t* vr = fresh ? a.v_new + kvrow * kD : a.v_res + (kvrow * a.residual_cap + slot) * kD;
        L.k0 = kr[lane];
        L.k1 = kr[lane + kRpPairs];
        L.v0 = vr[lane];
        L.v1 = vr[lane + kRpPairs];
    };
    RLoad nx;
    if (wave < rs.n_res) load(nx, wave);
    for (int i = wave; i < rs.n_res; i += kWaves) {
        const RLoad cur = nx;
        if (i + kWaves < rs.n_res) load(nx, i + kWaves);
        const float2 e = turn((double)(rs.n_quant + i) * wm);
        const float wr = fmaf(q0, e.x, q1 * e.y), wi = fmaf(q0, e.y, -q1 * e.x);   // conj(Q) * e
        const float part = fmaf(wr, h2f(cur.k0), -wi * h2f(cur.k1));
        const float lg = wave_sum(part) * a.sm_log2;
        const float mnew = fmaxf(mr, lg);
        const float al = mr == -INFINITY ? 0.0f : exp2_fast(mr - mnew);
        const float p = exp2_fast(lg - mnew);
        lr = fmaf(lr, al, p);
        o0 = fmaf(o0, al, p * h2f(cur.v0));
        o1 = fmaf(o1, al, p * h2f(cur.v1));
        mr = mnew;
    }
    o_dst[lane] = o0;
    o_dst[lane + kRpPairs] = o1;
}

// residual_rope_states for the NQ query heads qrow0..qrow0+NQ-1 of kv row kvrow: each key is
// turned once, R = K * exp(i*p*w) per pair (lane m: pair m), and head h's logit is the wave
// sum of Re(conj(Q_h) * R); the NQ sums are taken together (half_sum4, then one read of each
// half-wave per head).  States of head h go to o_dst[h], mr[h], lr[h].
template <int NQ>
__device__ void residual_rope_group_states(const AttnArgs& a, const RowState& rs, int64_t qrow0, int64_t kvrow, int wave,
                                           const double* w_pair, float* const (&o_dst)[NQ], float (&mr)[NQ], float (&lr)[NQ]) {
    static_assert(NQ <= 4, "up to four heads");
    const int lane = threadIdx.x & 63;
    float q0[NQ], q1[NQ], o0[NQ], o1[NQ];
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
        q0[h] = h2f(a.q[(qrow0 + h) * kD + lane]);
        q1[h] = h2f(a.q[(qrow0 + h) * kD + lane + kRpPairs]);
        o0[h] = o1[h] = 0.0f;
        mr[h] = -INFINITY;
        lr[h] = 0.0f;
    }
    const double wm = w_pair[lane];
    // the key and value channels lane, lane + 64 of residual token i, loaded a token ahead
    struct RLoad { uint16_t k0, k1, v0, v1; };
    auto load = [&](RLoad& L, int i) {
        const int slot = (rs.res_head + i) % a.residual_cap;
        const bool fresh = a.k_new != nullptr && i == rs.n_res - 1;
        const uint16_t* kr = fresh ? a.k_new + kvrow * kD : a.k_res + (kvrow * a.residual_cap + slot) * kD;
        const uint16_t* vr = fresh ? a.v_new + kvrow * kD : a.v_res + (kvrow * a.residual_cap + slot) * kD;
        L.k0 = kr[lane];
        L.k1 = kr[lane + kRpPairs];
        L.v0 = vr[lane];
        L.v1 = vr[lane + kRpPairs];
    };
    RLoad nx;
    if (wave < rs.n_res) load(nx, wave);
    for (int i = wave; i < rs.n_res; i += kWaves) {
        const RLoad cur = nx;
        if (i + kWaves < rs.n_res) load(nx, i + kWaves);
        const float2 e = turn((double)(rs.n_quant + i) * wm);
        const float k0 = h2f(cur.k0), k1 = h2f(cur.k1);
        const float rr = fmaf(k0, e.x, -k1 * e.y), ri = fmaf(k0, e.y, k1 * e.x);   // R = K * e
        float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < NQ; ++h) part[h] = fmaf(q0[h], rr, q1[h] * ri);
        // lane b0 + 2*b1 of each half-wave holds the half's sum of part[2*b0 + b1]
        const float x = half_sum4(part);
        const float v0 = h2f(cur.v0), v1 = h2f(cur.v1);
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
            const int src = (h >> 1) | ((h & 1) << 1);
            const float lg = (readlane_f(x, src) + readlane_f(x, 32 + src)) * a.sm_log2;
            const float mnew = fmaxf(mr[h], lg);
            const float al = mr[h] == -INFINITY ? 0.0f : exp2_fast(mr[h] - mnew);
            const float p = exp2_fast(lg - mnew);
            lr[h] = fmaf(lr[h], al, p);
            o0[h] = fmaf(o0[h], al, p * v0);
            o1[h] = fmaf(o1[h], al, p * v1);
            mr[h] = mnew;
        }
    }
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
        o_dst[h][lane] = o0[h];
        o_dst[h][lane + kRpPairs] = o1[h];
    }
}

template <int BITS, int GS, bool RAGGED>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void attn_rope_kernel(AttnArgs a) {
    constexpr int kIt = GS / kRpTok;   // iterations per key group
    __shared__ double sh_w[kRpPairs];                        // pair frequencies
    __shared__ __align__(16) float2 sh_ed[GS][kRpPairs];     // exp(i*d*w) for offsets d < G
    // the folded products U, V, X (real and imaginary parts) of the wave's group, per pair;
    // pair p at p + 4*(p/32), so that the eight 8-pair runs the lanes read at once start in
    // different 16-byte bank slots
    __shared__ __align__(16) float sh_f[kWaves][6][kRpPairs + 8];
    __shared__ __align__(16) float sh_p[kWaves][kRpTok];                // 4-bit: the iteration's weights
    // 2-bit values on the matrix cores: per wave the tile's 32 logits and its value weights
    // [channel group][32 tokens] (fp16, the A operand's weight row), and zero rows
    __shared__ __align__(16) float sh_lg[kWaves][kG];
    __shared__ __align__(16) uint8_t sh_wt[kWaves][4 * 64];
    __shared__ __align__(16) uint8_t sh_zr[4 * 64];
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

    // the query pair the lane folds once per group: channels lane and 64 + lane
    const float q_lo = h2f(a.q[qrow * kD + lane]), q_hi = h2f(a.q[qrow * kD + kRpPairs + lane]);

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
    // P.V lanes.  2-bit: per 32-token tile (every second iteration), on the matrix cores as
    // in the 2-bit kernels: lane l holds chunk l of the tile's value codes (the B operands of
    // all eight 16-channel blocks) and, for l < 32, token l's (scale, zero) pairs.
    // 4-bit: lane (vg, vc) reads tokens 4vg..4vg+3 and channels 8vc..8vc+7 (one group).
    constexpr int kVCh = BITS == 2 ? 1 : 8;               // channels per lane (4-bit)
    const int vg = lane >> 4, vc = lane & 15;
    struct VLoad { uint32_t c[4]; uint32_t p[4]; };
    auto load_v = [&](VLoad& L, int it) {
        if constexpr (BITS == 2) {
            // the tile of iteration it (past the end: the wave's last tile), so tokens
            // t0 + (lane & 31) are in the wave's groups
            const uint32_t t0 = (uint32_t)tok(it) & ~(uint32_t)(kG - 1);
            const uint4 x = reinterpret_cast<const uint4*>(vc_row + (t0 / kG) * kTileBytes)[lane];
            const uint4 y = load_value_pairs<GS, false>(vp_row + value_pair_index<GS>((int64_t)t0 + (lane & 31), 0));
            L.c[0] = x.x;
            L.c[1] = x.y;
            L.c[2] = x.z;
            L.c[3] = x.w;
            L.p[0] = y.x;
            L.p[1] = y.y;
            L.p[2] = y.z;
            L.p[3] = y.w;
        } else {
            const uint32_t t = (uint32_t)tok(it) + 4 * vg;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                L.c[u] = *reinterpret_cast<const uint32_t*>(vc_row + (t + u) * kRowBytes4 + 4 * vc);
                L.p[u] = vp_row[(t + u) * (kD / GS) + (8 * vc) / GS];
            }
        }
    };
    // key (scale, zero) words of group gi of the wave, channels lane and 64 + lane
    struct PLoad { uint32_t lo, hi; };
    auto load_kp = [&](PLoad& L, int gi) {
        const uint32_t* g = kp_row + (int64_t)(kgb + min(gi, n_groups - 1)) * kD;
        L.lo = g[lane];
        L.hi = g[kRpPairs + lane];
    };
    auto wave_sync = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    float m = -INFINITY, lsum = 0.0f, o[kVCh], oz = 0.0f;   // o, oz: 4-bit, the lane's channels and its tokens' p*z
#pragma unroll
    for (int c = 0; c < kVCh; ++c) o[c] = 0.0f;
    float* pw = &sh_p[wave][0];
    // 2-bit: accumulators of the eight 16-channel blocks, block v in row v%4 of cv[v/4] (its
    // A operand has the weights in that row, zeros elsewhere); p*zero per 32-channel group;
    // vs, a power of two keeping the fp16 weights in range.  Lane l < 32 takes token l of a
    // tile for the weights, whose A-operand slots order tokens 8kg..8kg+7 as 0,4,1,5,2,6,3,7
    // (the order the masked code fields produce them in); token 4a + i meets its code as the
    // fp16 subnormal c * 4^i * 2^-24, so its weight carries 16 * 4^-i.
    v4f cv[2] = {(v4f){0.0f, 0.0f, 0.0f, 0.0f}, (v4f){0.0f, 0.0f, 0.0f, 0.0f}};
    float zk[4] = {0.0f, 0.0f, 0.0f, 0.0f}, vs = 0.0f;
    uint8_t* wt = &sh_wt[wave][0];
    if (BITS == 2 && threadIdx.x < 16) reinterpret_cast<uint4*>(sh_zr)[threadIdx.x] = make_uint4(0, 0, 0, 0);

    KLoad kl;
    VLoad vl;
    PLoad pn;
    if (n_groups > 0) {   // the first iteration's loads, in flight while the turn tables are built
        load_k(kl, 0);
        if constexpr (BITS != 2) load_v(vl, 0);
        load_kp(pn, 0);
    }
    // pair frequencies and the in-group turns exp(i*d*w)
    if (threadIdx.x < kRpPairs) sh_w[threadIdx.x] = pow(a.rope_base, -2.0 * (double)threadIdx.x / (double)kD);
    __syncthreads();
    for (int i = threadIdx.x; i < GS * kRpPairs; i += kBlock) sh_ed[i / kRpPairs][i % kRpPairs] = turn((double)(i / kRpPairs) * sh_w[i % kRpPairs]);
    __syncthreads();

    uint32_t tag;
    if (n_groups > 0) {
        GroupTurn gt;
        gt.init(sh_w[lane], GS);   // the frequency of the lane's pair
        const int f_slot = lane + 4 * (lane >> 5), f_run = 8 * k8 + 4 * (k8 >> 2);
        tag = settle_tag(tag_v);
        for (int gi = 0; gi < n_groups; ++gi) {
            set_priority_for(n_groups - gi);   // (as in the query-group kernel: most work left issues first)
            // ---- the group's folded products, pair = lane: each is needed by the 8 lanes that
            // take the pair's channels, so it is formed once and shared through LDS
            {
                const float2 e = gt.next(gi, (int64_t)(kgb + gi) * GS);   // exp(i*t0*w)
                const float wr = fmaf(q_lo, e.x, q_hi * e.y);    // W = conj(Q) * e
                const float wi = fmaf(q_lo, e.y, -q_hi * e.x);
                const float slo = h2f(pn.lo & 0xffffu), zlo = h2f(pn.lo >> 16);
                const float shi = h2f(pn.hi & 0xffffu), zhi = h2f(pn.hi >> 16);
                float(*f)[kRpPairs + 8] = sh_f[wave];
                f[0][f_slot] = fmaf(wr, zlo, -wi * zhi);   // U = W * (zlo + i*zhi)
                f[1][f_slot] = fmaf(wr, zhi, wi * zlo);
                f[2][f_slot] = wr * slo;                   // V = W * slo
                f[3][f_slot] = wi * slo;
                f[4][f_slot] = -wi * shi;                  // X = i * W * shi
                f[5][f_slot] = wr * shi;
            }
            load_kp(pn, gi + 1);
            wave_sync();
            // the lane's pairs 8k8..8k8+7
            float ur[8], ui[8], vr[8], vi[8], xr[8], xi[8];
            {
                auto run = [&](int c, float (&d)[8]) {
                    const float4 lo = *reinterpret_cast<const float4*>(&sh_f[wave][c][f_run]);
                    const float4 hi = *reinterpret_cast<const float4*>(&sh_f[wave][c][f_run + 4]);
                    d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
                    d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
                };
                run(0, ur); run(1, ui); run(2, vr); run(3, vi); run(4, xr); run(5, xi);
            }
            wave_sync();   // every lane has read the products before the next group's are written
            // (unrolled by two: a tile's even and odd iterations have code of their own, so the
            // tile's value loads, issued at the top of its odd iteration, are live for one)
#pragma unroll 2
            for (int j = 0; j < kIt; ++j) {
                const int it = gi * kIt + j;
                if constexpr (BITS == 2) {
                    if (j & 1) load_v(vl, it);
                }
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
                float mx = fmax_ieee(lg[0], lg[1]);
                mx = fmax_ieee(mx, perm_f<0x128>(mx));   // lane (i+8)%16 of the row
                mx = fmax_ieee(mx, xor16_f(mx));
                mx = fmax_ieee(readlane_f(mx, 0), readlane_f(mx, 32));
                const float mnew = fmax_ieee(m, mx);
                if (mnew != m) {
                    const float al = m == -INFINITY ? 0.0f : exp2_fast(m - mnew);
                    if constexpr (BITS == 2) {
                        cv[0] *= al;
                        cv[1] *= al;
#pragma unroll
                        for (int k = 0; k < 4; ++k) zk[k] *= al;
                    } else {
#pragma unroll
                        for (int c = 0; c < kVCh; ++c) o[c] *= al;
                        oz *= al;
                    }
                    lsum *= al;
                    m = mnew;
                }
                if constexpr (BITS == 2) {
                    // logits of the tile's tokens 16(j%2) + t8 and 16(j%2) + 8 + t8
                    if (k8 == 0) {
                        sh_lg[wave][16 * (j & 1) + t8] = lg[0];
                        sh_lg[wave][16 * (j & 1) + 8 + t8] = lg[1];
                    }
                } else {
                    const float p0 = exp2_fast(lg[0] - m), p1 = exp2_fast(lg[1] - m);
                    if (k8 == 0) {
                        lsum += p0 + p1;
                        pw[t8] = p0;
                        pw[8 + t8] = p1;
                    }
                }
                wave_sync();
                // ---- P.V, dequantization folded: (p*s)*c + p*z
                if constexpr (BITS == 2) {
                    if (j & 1) {   // the tile's 32 logits are in: its weights, then 8 matrix instructions
                        const int tt = lane & 31, mrow = lane & 15, kgrp = lane >> 4;
                        const float p = lane < kG ? exp2_fast(sh_lg[wave][tt] - m) : 0.0f;   // token tt (lanes < 32)
                        lsum += p;
#pragma unroll
                        for (int k = 0; k < 4; ++k) zk[k] = fmaf(p, h2f(vl.p[k] >> 16), zk[k]);
                        // the largest scale, on the fp16 bit patterns (scales are never negative)
                        const float smax = lane < kG ? h2f(max_u16x2(max_u16x2(vl.p[0], vl.p[1]), max_u16x2(vl.p[2], vl.p[3])) & 0xffffu) : 0.0f;
                        // weights 16*p*s*vs must stay below 2^15: shrink vs (a power of two) if needed
                        if (__builtin_amdgcn_ballot_w64(smax * vs > 2048.0f || vs == 0.0f)) {
                            const float gm = wave_max_xor(smax, 1, 32);
                            const float nvs = __builtin_ldexpf(1.0f, 11 - __builtin_amdgcn_frexp_expf(gm));
                            if (vs != 0.0f && nvs < vs) {
                                const float r = nvs / vs;
                                cv[0] *= r;
                                cv[1] *= r;
                            }
                            if (vs == 0.0f || nvs < vs) vs = nvs;
                        }
                        if (lane < kG) {
                            const int w_off = (tt >> 3) * 16 + (((tt & 3) << 1) | ((tt >> 2) & 1)) * 2;
                            const float f = p * (__builtin_ldexpf(16.0f, -2 * (tt & 3)) * vs);
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                *reinterpret_cast<_Float16*>(wt + w_off + k * 64) = (_Float16)(f * h2f(vl.p[k] & 0xffffu));
                        }
                        wave_sync();
                        constexpr uint32_t kF0 = 0x00030003u, kF1 = 0x000C000Cu, kF2 = 0x00300030u, kF3 = 0x00C000C0u;
#pragma unroll
                        for (int v = 0; v < 8; ++v) {
                            // word v/2 holds blocks v (even) and v+1 in alternate bytes; token field
                            // i of each byte, masked in place, is the fp16 subnormal c * 4^i * 2^-24
                            const uint32_t x = (v & 1) ? vl.c[v >> 1] >> 8 : vl.c[v >> 1];
                            const v8h bop = __builtin_bit_cast(v8h, make_uint4(x & kF0, x & kF1, x & kF2, x & kF3));
                            const uint8_t* arow = (mrow == (v & 3) ? wt : sh_zr) + (v >> 1) * 64 + 16 * kgrp;
                            const v8h aop = *reinterpret_cast<const v8h*>(arow);
                            cv[v >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, cv[v >> 2], 0, 0, 0);
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
                    load_v(vl, it + 1);
                }
                wave_sync();
            }
        }
    } else {
        tag = settle_tag(tag_v);
    }

    // ---- the wave's state: p*z shares added to their channels, lanes of a channel summed
    if constexpr (BITS == 2) {
        // o = P.V * 2^20 / vs + sum p*zero; block v's row sits in row v%4 of cv[v/4] (lanes 0..15)
#pragma unroll
        for (int k = 0; k < 4; ++k) zk[k] = wave_sum(zk[k]);
        const float inv = vs != 0.0f ? 1048576.0f / vs : 0.0f;
        if (lane < 16) {
#pragma unroll
            for (int v = 0; v < 8; ++v) sh_o[0][wave][16 * v + lane] = fmaf(cv[v >> 2][v & 3], inv, zk[v >> 1]);
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
    __builtin_amdgcn_s_setprio(0);
    if (split == rs.res_split) {
        __builtin_amdgcn_s_setprio(2);   // the residual is work the other splits do not have
        residual_rope_states(a, rs, qrow, kvrow, wave, sh_w, &sh_o[0][kWaves + wave][0], mr, lr);
        __builtin_amdgcn_s_setprio(0);
    }
    if (lane == 0) {
        sh_m[0][kWaves + wave] = mr;
        sh_l[0][kWaves + wave] = lr;
    }
    __syncthreads();
    finish_block<1>(a, rs.splits, split, qrow, tag, sh_o, sh_m, sh_l);
}

// Query-group form: the NQ query heads qrow0..qrow0+NQ-1
// of one kv head in one workgroup, which dequantizes and turns each key once for all of them.
// The group's folded products then carry no query: with E0 = exp(i*t0*w), U = E0*(z_i +
// i*z_{i+64}), V = E0*s_i and X = i*E0*s_{i+64}, a token's turned key pair is R = (U + V*c +
// X*c') * exp(i*d*w) (four fmas and a complex product), and head h adds Re(conj(Q_h)*R) =
// q_{h,i}*Re R + q_{h,i+64}*Im R (two fmas) to its logit: 10 + 2*NQ operations per pair and
// token with the two code conversions, against 8 for each head in a workgroup of its own.
// A lane's 2*NQ partial logits per 16 tokens (two tokens, NQ heads) are summed over the
// token's 8 lanes by halving exchanges (token_head_sums), after which each lane holds one
// (token, head) sum.  2-bit P.V shares each value tile's 8 matrix instructions among the
// heads: head h's weights go in row 4*(v%4) + h of block v's A operand, so that the
// accumulators' register h is head h.  4-bit P.V runs on the vector units as in the one-head
// kernel, each lane's value codes converted once for all heads; every lane forms the weight
// of the (token, head) sum it holds and passes it through LDS.

// Sums over the 8 lanes of a token (k8 = lane & 7) of 2*NQ values, v[ps][h] = token ps's
// partial logit of head h.  Each step a lane keeps half of its values and adds its partner's
// copies of them, while the partner keeps the other half: partners k8 ^ 7 (the half-row
// mirror), then k8 ^ 1, then k8 ^ 2 (for two heads a plain sum over k8 ^ 2).  Index n = 2h + ps
// ends in the lane with n = k8 (four heads) or n = 2*(k8 >> 2) + (k8 & 1) (two heads).
template <int NQ>
__device__ __forceinline__ float token_head_sums(const float (&v)[2][NQ], int k8) {
    const bool b0 = k8 & 1, b1 = k8 & 2, b2 = k8 & 4;
    if constexpr (NQ == 4) {
        float w[4];   // w[m]: index m + 4*b2
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float lo = v[m & 1][m >> 1], hi = v[m & 1][(m >> 1) + 2];
            w[m] = (b2 ? hi : lo) + hmirror_f(b2 ? lo : hi);
        }
        float x[2];   // x[u]: index 4*b2 + 2u + b0
#pragma unroll
        for (int u = 0; u < 2; ++u) x[u] = (b0 ? w[2 * u + 1] : w[2 * u]) + xor1_f(b0 ? w[2 * u] : w[2 * u + 1]);
        return (b1 ? x[1] : x[0]) + xor2_f(b1 ? x[0] : x[1]);
    } else {
        float w[2];   // w[m]: index m + 2*b2
#pragma unroll
        for (int m = 0; m < 2; ++m) w[m] = (b2 ? v[m][1] : v[m][0]) + hmirror_f(b2 ? v[m][0] : v[m][1]);
        const float x = (b0 ? w[1] : w[0]) + xor1_f(b0 ? w[0] : w[1]);
        return x + xor2_f(x);
    }
}

template <int BITS, int GS, int NQ, bool RAGGED>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(GS == 128 ? 1 : 2))) void attn_rope_group_kernel(AttnArgs a) {
    static_assert(NQ >= 2 && NQ <= 4, "two to four query heads per workgroup");
    constexpr int kIt = GS / kRpTok;   // iterations per key group
    // heads as the lanes see them: three take the four-head layout, the fourth head idle (its
    // queries zero, its sums and weights never used)
    constexpr int NP = NQ == 2 ? 2 : 4;
    constexpr int NH = NP / 2;         // 2-bit P.V weights: heads per lane, lane >> 5 picks which
    __shared__ double sh_w[kRpPairs];
    __shared__ __align__(16) float2 sh_ed[GS][kRpPairs];
    __shared__ __align__(16) float sh_f[kWaves][6][kRpPairs + 8];
    __shared__ __align__(16) float sh_lg[kWaves][NP][kG];
    __shared__ __align__(16) uint8_t sh_wt[kWaves][NP][4 * 64];
    __shared__ __align__(16) uint8_t sh_zr[4 * 64];
    __shared__ __align__(16) float sh_p[kWaves][NP][kRpTok];   // 4-bit: the iteration's weights
    __shared__ __align__(16) float sh_o[NQ][kSlots][kD];
    __shared__ float sh_m[NQ][kSlots], sh_l[NQ][kSlots];

    // (ragged batch: the plan uses sh_o, unused until the end)
    const WorkItem wi = work_item<RAGGED>(a, reinterpret_cast<int32_t*>(&sh_o[0][0][0]));
    if (RAGGED && wi.split < 0) return;   // (ragged batch) past the plan's last item
    const int split = wi.split;
    const int64_t qrow0 = wi.row * NQ;   // grid row = kvrow*(ratio/NQ) + chunk
    const int64_t kvrow = (int64_t)((uint32_t)qrow0 / (uint32_t)a.ratio);
    if (a.k_new != nullptr && split == 0 && (uint32_t)qrow0 % (uint32_t)a.ratio == 0) store_new_token(a, kvrow);
    const TagLoads<NQ> tag_v = partial_tag<NQ>(a, qrow0);
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

    // the lane's pairs 8k8..8k8+7 of every head: Q = q_i + i*q_{i+64}
    float qr[NQ][8], qi[NQ][8];
#pragma unroll
    for (int h = 0; h < NQ; ++h)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            qr[h][jj] = h2f(a.q[(qrow0 + h) * kD + 8 * k8 + jj]);
            qi[h][jj] = h2f(a.q[(qrow0 + h) * kD + kRpPairs + 8 * k8 + jj]);
        }

    const int64_t tok0 = kvrow * (int64_t)a.token_cap;
    const uint8_t* kc_row = a.k_codes + tok0 * (BITS == 2 ? kRowBytes : kRowBytes4);
    const uint8_t* vc_row = a.v_codes + tok0 * (BITS == 2 ? kRowBytes : kRowBytes4);
    const uint32_t* kp_row = reinterpret_cast<const uint32_t*>(a.k_sz) + kvrow * (int64_t)(a.token_cap / GS) * kD;
    const uint32_t* vp_row = reinterpret_cast<const uint32_t*>(a.v_sz) + tok0 * (kD / GS);
    const int t_b = kgb * GS;
    auto tok = [&](int it) { return t_b + min(it, n_it - 1) * kRpTok; };   // clamped past the end

    // key codes of the two pass tokens, as in the one-head kernel
    struct KLoad { uint32_t lo[2], hi[2]; };
    auto load_k = [&](KLoad& L, int it) {
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const uint32_t t = (uint32_t)(tok(it) + 8 * ps + t8);
            if constexpr (BITS == 2) {
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
    // 2-bit: the value tile of iteration it, lane l holding chunk l of the codes and token
    // l % 32's pairs.  4-bit: lane (vg, vc) reads tokens 4vg..4vg+3 of the iteration and
    // channels 8vc..8vc+7, as in the one-head kernel.
    const int vg = lane >> 4, vc = lane & 15;
    struct VLoad { uint32_t c[4]; uint32_t p[4]; };
    auto load_v = [&](VLoad& L, int it) {
        if constexpr (BITS == 2) {
            const uint32_t t0 = (uint32_t)tok(it) & ~(uint32_t)(kG - 1);
            const uint4 x = reinterpret_cast<const uint4*>(vc_row + (t0 / kG) * kTileBytes)[lane];
            const uint4 y = load_value_pairs<GS, false>(vp_row + value_pair_index<GS>((int64_t)t0 + (lane & 31), 0));
            L.c[0] = x.x;
            L.c[1] = x.y;
            L.c[2] = x.z;
            L.c[3] = x.w;
            L.p[0] = y.x;
            L.p[1] = y.y;
            L.p[2] = y.z;
            L.p[3] = y.w;
        } else {
            const uint32_t t = (uint32_t)tok(it) + 4 * vg;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                L.c[u] = *reinterpret_cast<const uint32_t*>(vc_row + (t + u) * kRowBytes4 + 4 * vc);
                L.p[u] = vp_row[(t + u) * (kD / GS) + (8 * vc) / GS];
            }
        }
    };
    struct PLoad { uint32_t lo, hi; };
    auto load_kp = [&](PLoad& L, int gi) {
        const uint32_t* g = kp_row + (int64_t)(kgb + min(gi, n_groups - 1)) * kD;
        L.lo = g[lane];
        L.hi = g[kRpPairs + lane];
    };
    auto wave_sync = []() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // running maxima (wave-uniform), P.V accumulators (register h: head h), and per lane the
    // sums and p*zero shares of heads NH*(lane >> 5) + u
    float m[NP];
#pragma unroll
    for (int h = 0; h < NP; ++h) m[h] = -INFINITY;
    v4f cv[2] = {(v4f){0.0f, 0.0f, 0.0f, 0.0f}, (v4f){0.0f, 0.0f, 0.0f, 0.0f}};
    float zk[NH][4], ls[NH], vs = 0.0f;
#pragma unroll
    for (int u = 0; u < NH; ++u) {
        ls[u] = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) zk[u][k] = 0.0f;
    }
    const bool hp = lane >= 32;
    // 4-bit: the lane's channels of every head, and their p*zero share; the sum of the
    // weights of the (token, head) sums the lane holds (head h_lane below)
    float o4[NQ][8], oz4[NQ], ls4 = 0.0f;
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
        oz4[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o4[h][c] = 0.0f;
    }
    if (BITS == 2 && threadIdx.x < 16) reinterpret_cast<uint4*>(sh_zr)[threadIdx.x] = make_uint4(0, 0, 0, 0);

    KLoad kl;
    VLoad vl;
    PLoad pn;
    if (n_groups > 0) {
        load_k(kl, 0);
        if constexpr (BITS != 2) load_v(vl, 0);
        load_kp(pn, 0);
    }
    if (threadIdx.x < kRpPairs) sh_w[threadIdx.x] = pow(a.rope_base, -2.0 * (double)threadIdx.x / (double)kD);
    __syncthreads();
    for (int i = threadIdx.x; i < GS * kRpPairs; i += kBlock) sh_ed[i / kRpPairs][i % kRpPairs] = turn((double)(i / kRpPairs) * sh_w[i % kRpPairs]);
    __syncthreads();

    uint32_t tag;
    if (n_groups > 0) {
        GroupTurn gt;
        gt.init(sh_w[lane], GS);
        const int f_slot = lane + 4 * (lane >> 5), f_run = 8 * k8 + 4 * (k8 >> 2);
        const int h_lane = NP == 4 ? k8 >> 1 : k8 >> 2;   // the (token, head) sum a lane ends with
        const bool lg_store = (NP == 4 || (k8 & 2) == 0) && h_lane < NQ;
        tag = settle_tag(tag_v);
        for (int gi = 0; gi < n_groups; ++gi) {
            set_priority_for(n_groups - gi);
            {
                const float2 e = gt.next(gi, (int64_t)(kgb + gi) * GS);   // E0 = exp(i*t0*w)
                const float slo = h2f(pn.lo & 0xffffu), zlo = h2f(pn.lo >> 16);
                const float shi = h2f(pn.hi & 0xffffu), zhi = h2f(pn.hi >> 16);
                float(*f)[kRpPairs + 8] = sh_f[wave];
                f[0][f_slot] = fmaf(e.x, zlo, -e.y * zhi);   // U = E0 * (zlo + i*zhi)
                f[1][f_slot] = fmaf(e.x, zhi, e.y * zlo);
                f[2][f_slot] = e.x * slo;                    // V = E0 * slo
                f[3][f_slot] = e.y * slo;
                f[4][f_slot] = -e.y * shi;                   // X = i * E0 * shi
                f[5][f_slot] = e.x * shi;
            }
            load_kp(pn, gi + 1);
            wave_sync();
            float ur[8], ui[8], vr[8], vi[8], xr[8], xi[8];
            {
                auto run = [&](int c, float (&d)[8]) {
                    const float4 lo = *reinterpret_cast<const float4*>(&sh_f[wave][c][f_run]);
                    const float4 hi = *reinterpret_cast<const float4*>(&sh_f[wave][c][f_run + 4]);
                    d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
                    d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
                };
                run(0, ur); run(1, ui); run(2, vr); run(3, vi); run(4, xr); run(5, xi);
            }
            wave_sync();
#pragma unroll 2
            for (int j = 0; j < kIt; ++j) {
                const int it = gi * kIt + j;
                if constexpr (BITS == 2) {
                    if (j & 1) load_v(vl, it);
                }
                // ---- partial logits of tokens t8 and 8 + t8, the lane's 8 pairs, every head
                float part[2][NP];
#pragma unroll
                for (int ps = 0; ps < 2; ++ps) {
                    float c1[8], c2[8];
                    codes8<BITS>(kl.lo[ps], k8 & 1, c1);
                    codes8<BITS>(kl.hi[ps], k8 & 1, c2);
                    const float2* ed = &sh_ed[kRpTok * j + 8 * ps + t8][8 * k8];
#pragma unroll
                    for (int h = 0; h < NP; ++h) part[ps][h] = 0.0f;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const float2 e = ed[jj];
                        const float kr = fmaf(xr[jj], c2[jj], fmaf(vr[jj], c1[jj], ur[jj]));
                        const float ki = fmaf(xi[jj], c2[jj], fmaf(vi[jj], c1[jj], ui[jj]));
                        const float rr = fmaf(kr, e.x, -ki * e.y);   // R = (kr + i*ki) * exp(i*d*w)
                        const float ri = fmaf(kr, e.y, ki * e.x);
#pragma unroll
                        for (int h = 0; h < NQ; ++h) part[ps][h] = fmaf(qr[h][jj], rr, fmaf(qi[h][jj], ri, part[ps][h]));
                    }
                }
                load_k(kl, it + 1);
                const float lg = token_head_sums<NP>(part, k8) * a.sm_log2;   // token 8(k8&1) + t8, head h_lane
                if (BITS == 2 && lg_store) sh_lg[wave][h_lane][16 * (j & 1) + 8 * (k8 & 1) + t8] = lg;
                // ---- running maxima: over the lanes that hold a head's 16 sums, then per head
                float mx = fmax_ieee(lg, perm_f<0xB1>(lg));
                if constexpr (NP == 2) mx = fmax_ieee(mx, perm_f<0x4E>(mx));
                mx = fmax_ieee(mx, perm_f<0x128>(mx));   // lane (i+8)%16 of the row
                mx = fmax_ieee(mx, xor16_f(mx));
                float al[NP];
                bool moved = false;
#pragma unroll
                for (int h = NQ; h < NP; ++h) al[h] = 1.0f;
#pragma unroll
                for (int h = 0; h < NQ; ++h) {
                    const int src = NP == 4 ? 2 * h : 4 * h;
                    const float mnew = fmax_ieee(m[h], fmax_ieee(readlane_f(mx, src), readlane_f(mx, 32 + src)));
                    al[h] = mnew == m[h] ? 1.0f : (m[h] == -INFINITY ? 0.0f : exp2_fast(m[h] - mnew));
                    moved |= mnew != m[h];
                    m[h] = mnew;
                }
                if (moved) {
                    if constexpr (BITS == 2) {
#pragma unroll
                        for (int h = 0; h < NQ; ++h) {
                            cv[0][h] *= al[h];
                            cv[1][h] *= al[h];
                        }
#pragma unroll
                        for (int u = 0; u < NH; ++u) {
                            const float a_u = hp ? al[NH + u] : al[u];
                            ls[u] *= a_u;
#pragma unroll
                            for (int k = 0; k < 4; ++k) zk[u][k] *= a_u;
                        }
                    } else {
                        float a_l = al[0];   // the factor of the lane's own head
#pragma unroll
                        for (int h = 1; h < NQ; ++h) a_l = h_lane == h ? al[h] : a_l;
                        ls4 *= a_l;
#pragma unroll
                        for (int h = 0; h < NQ; ++h) {
                            oz4[h] *= al[h];
#pragma unroll
                            for (int c = 0; c < 8; ++c) o4[h][c] *= al[h];
                        }
                    }
                }
                if constexpr (BITS != 2) {
                    // the weight of the lane's (token, head) sum, into LDS for the P.V lanes
                    float m_l = m[0];
#pragma unroll
                    for (int h = 1; h < NQ; ++h) m_l = h_lane == h ? m[h] : m_l;
                    const float p = exp2_fast(lg - m_l);
                    if (lg_store) {
                        ls4 += p;
                        sh_p[wave][h_lane][8 * (k8 & 1) + t8] = p;
                    }
                }
                wave_sync();
                // ---- P.V: 2-bit, of the tile once its 32 logits are in; 4-bit, of the
                // iteration's 16 tokens on the vector units, (p*s)*c + p*z
                if constexpr (BITS != 2) {
                    // Two tokens per instruction: v_dot2_f32_f16 of the pair's weights
                    // p*s*vs (fp16) with their codes of one channel, placed in the low bits of
                    // each half as the fp16 subnormals c * 2^-24 (channel 2b) and 16c * 2^-24
                    // (2b + 1), no conversion.  vs, a power of two shared by the wave, keeps
                    // the weights below 2^14.
                    float smax = 0.0f;
#pragma unroll
                    for (int u = 0; u < 4; ++u) smax = fmaxf(smax, h2f(vl.p[u] & 0xffffu));
                    if (__builtin_amdgcn_ballot_w64(smax * vs > 16384.0f || (vs == 0.0f && smax > 0.0f))) {
                        const float gm = wave_max_xor(smax, 1, 32);
                        const float nvs = __builtin_ldexpf(1.0f, 14 - __builtin_amdgcn_frexp_expf(gm));
                        if (vs != 0.0f && nvs < vs) {
                            const float r = nvs / vs;
#pragma unroll
                            for (int h = 0; h < NQ; ++h)
#pragma unroll
                                for (int c = 0; c < 8; ++c) o4[h][c] *= r;
                        }
                        if (vs == 0.0f || nvs < vs) vs = nvs;
                    }
                    uint32_t cl[2][4], ch[2][4];   // [token pair][byte]: channels 8vc + 2b, 8vc + 2b + 1
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            // byte b of the pair's first word in byte 0, of its second in byte 2
                            const uint32_t x = __builtin_amdgcn_perm(vl.c[2 * j + 1], vl.c[2 * j], 0x0C000C00u | ((4u + b) << 16) | b);
                            cl[j][b] = x & 0x000F000Fu;
                            ch[j][b] = x & 0x00F000F0u;
                        }
                    float sv[4], zv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        sv[u] = h2f(vl.p[u] & 0xffffu) * vs;
                        zv[u] = h2f(vl.p[u] >> 16);
                    }
#pragma unroll
                    for (int h = 0; h < NQ; ++h) {
                        const float4 pt = *reinterpret_cast<const float4*>(&sh_p[wave][h][4 * vg]);
                        oz4[h] = fmaf(pt.x, zv[0], fmaf(pt.y, zv[1], fmaf(pt.z, zv[2], fmaf(pt.w, zv[3], oz4[h]))));
                        const h2v w0 = {(_Float16)(pt.x * sv[0]), (_Float16)(pt.y * sv[1])};
                        const h2v w1 = {(_Float16)(pt.z * sv[2]), (_Float16)(pt.w * sv[3])};
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            o4[h][2 * b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, cl[0][b]), w0, o4[h][2 * b], false);
                            o4[h][2 * b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, cl[1][b]), w1, o4[h][2 * b], false);
                            o4[h][2 * b + 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, ch[0][b]), w0, o4[h][2 * b + 1], false);
                            o4[h][2 * b + 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, ch[1][b]), w1, o4[h][2 * b + 1], false);
                        }
                    }
                    load_v(vl, it + 1);
                } else if (j & 1) {
                    const int tt = lane & 31, mrow = lane & 15, kgrp = lane >> 4;
                    float p[NH];
#pragma unroll
                    for (int u = 0; u < NH; ++u) {
                        const float mh = hp ? m[NH + u] : m[u];
                        p[u] = NH * (int)hp + u < NQ ? exp2_fast(sh_lg[wave][NH * (int)hp + u][tt] - mh) : 0.0f;
                        ls[u] += p[u];
#pragma unroll
                        for (int k = 0; k < 4; ++k) zk[u][k] = fmaf(p[u], h2f(vl.p[k] >> 16), zk[u][k]);
                    }
                    const float smax = h2f(max_u16x2(max_u16x2(vl.p[0], vl.p[1]), max_u16x2(vl.p[2], vl.p[3])) & 0xffffu);
                    if (__builtin_amdgcn_ballot_w64(smax * vs > 2048.0f || vs == 0.0f)) {
                        const float gm = wave_max_xor(smax, 1, 32);
                        const float nvs = __builtin_ldexpf(1.0f, 11 - __builtin_amdgcn_frexp_expf(gm));
                        if (vs != 0.0f && nvs < vs) {
                            const float r = nvs / vs;
                            cv[0] *= r;
                            cv[1] *= r;
                        }
                        if (vs == 0.0f || nvs < vs) vs = nvs;
                    }
                    const int w_off = (tt >> 3) * 16 + (((tt & 3) << 1) | ((tt >> 2) & 1)) * 2;
                    const float sc = __builtin_ldexpf(16.0f, -2 * (tt & 3)) * vs;
#pragma unroll
                    for (int u = 0; u < NH; ++u) {
                        uint8_t* wt = &sh_wt[wave][NH * (int)hp + u][0];
                        const float f = p[u] * sc;
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            *reinterpret_cast<_Float16*>(wt + w_off + k * 64) = (_Float16)(f * h2f(vl.p[k] & 0xffffu));
                    }
                    wave_sync();
                    constexpr uint32_t kF0 = 0x00030003u, kF1 = 0x000C000Cu, kF2 = 0x00300030u, kF3 = 0x00C000C0u;
                    const int hr = mrow & 3;
                    const uint8_t* wrow = hr < NQ ? &sh_wt[wave][hr < NQ ? hr : 0][0] : sh_zr;
#pragma unroll
                    for (int v = 0; v < 8; ++v) {
                        const uint32_t x = (v & 1) ? vl.c[v >> 1] >> 8 : vl.c[v >> 1];
                        const v8h bop = __builtin_bit_cast(v8h, make_uint4(x & kF0, x & kF1, x & kF2, x & kF3));
                        const uint8_t* arow = ((mrow >> 2) == (v & 3) ? wrow : sh_zr) + (v >> 1) * 64 + 16 * kgrp;
                        const v8h aop = *reinterpret_cast<const v8h*>(arow);
                        cv[v >> 2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, cv[v >> 2], 0, 0, 0);
                    }
                }
                wave_sync();
            }
        }
    } else {
        tag = settle_tag(tag_v);
    }

    // ---- the wave's states.  2-bit: o = P.V * 2^20 / vs + sum p*zero; lane l holds channels
    // 16g + c and 16(g + 4) + c (g = l >> 4, c = l & 15) of every head.  4-bit: lanes of a
    // channel run summed (over the token quads), each head's weight sums over the lanes that
    // held its (token, head) sums.
    if constexpr (BITS != 2) {
        // o = P.V * 2^24 / vs (odd channels 2^20 / vs: their codes sat 4 bits higher) + sum p*z
        const float inv = vs != 0.0f ? 16777216.0f / vs : 0.0f;
        float v = ls4 + __shfl_xor(ls4, 1, 64);
        if constexpr (NP == 2) v += __shfl_xor(v, 2, 64);
        v = wave_sum_xor(v, 8, 32);
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float x = fmaf(o4[h][c], (c & 1) ? inv * 0.0625f : inv, oz4[h]);
                x += xor16_f(x);
                x += __shfl_xor(x, 32, 64);   // the four token quads (vg)
                if (lane < 16) sh_o[h][wave][8 * vc + c] = x;
            }
            const float lt = readlane_f(v, NP == 4 ? 2 * h : 4 * h);
            if (lane == 0) {
                sh_m[h][wave] = n_groups > 0 ? m[h] : -INFINITY;
                sh_l[h][wave] = lt;
            }
        }
    } else {
        float zt[NP][4], lt[NP];
#pragma unroll
        for (int u = 0; u < NH; ++u) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float s = wave_sum_xor(zk[u][k], 1, 16);   // over each half-wave
                zt[u][k] = readlane_f(s, 0);
                zt[NH + u][k] = readlane_f(s, 32);
            }
            const float s = wave_sum_xor(ls[u], 1, 16);
            lt[u] = readlane_f(s, 0);
            lt[NH + u] = readlane_f(s, 32);
        }
        const float inv = vs != 0.0f ? 1048576.0f / vs : 0.0f;
        const int g = lane >> 4, c = lane & 15;
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
            sh_o[h][wave][16 * g + c] = fmaf(cv[0][h], inv, zt[h][g >> 1]);
            sh_o[h][wave][16 * (g + 4) + c] = fmaf(cv[1][h], inv, zt[h][(g + 4) >> 1]);
            if (lane == 0) {
                sh_m[h][wave] = n_groups > 0 ? m[h] : -INFINITY;
                sh_l[h][wave] = lt[h];
            }
        }
    }
    // ---- fp16 residual (split rs.res_split), keys turned at n_quant + i once for all heads
    __builtin_amdgcn_s_setprio(0);
    {
        float mr[NQ], lr[NQ];
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
            mr[h] = -INFINITY;
            lr[h] = 0.0f;
        }
        if (split == rs.res_split) {
            __builtin_amdgcn_s_setprio(2);
            float* dst[NQ];
#pragma unroll
            for (int h = 0; h < NQ; ++h) dst[h] = &sh_o[h][kWaves + wave][0];
            residual_rope_group_states<NQ>(a, rs, qrow0, kvrow, wave, sh_w, dst, mr, lr);
            __builtin_amdgcn_s_setprio(0);
        }
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
                sh_m[h][kWaves + wave] = mr[h];
                sh_l[h][kWaves + wave] = lr[h];
            }
        }
    }
    __syncthreads();
    finish_block<NQ>(a, rs.splits, split, qrow0, tag, sh_o, sh_m, sh_l);
}

hipError_t launch_decode_attn_rope(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = attn_grid(a, a.q_rows);
#define KIVI_ROPE(BITSv, RAGGEDv)                                                                                  \
    KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_rope_kernel<BITSv, GS, RAGGEDv>), grid, dim3(kBlock), 0, s, t0, t1, \
                                                 0, a))
    const bool ragged = a.seq_state != nullptr;
    if (a.nq > 1) {
        const dim3 ggrid = attn_grid(a, a.block_rows);
#define KIVI_ROPE_GROUP(BITSv, NQv)                                                                                 \
    if (ragged)                                                                                                      \
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_rope_group_kernel<BITSv, GS, NQv, true>), ggrid, dim3(kBlock), \
                                                     0, s, t0, t1, 0, a))                                           \
    else                                                                                                             \
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_rope_group_kernel<BITSv, GS, NQv, false>), ggrid, dim3(kBlock), \
                                                     0, s, t0, t1, 0, a))
        if (a.bits == 4) {
            if (a.nq == 4) { KIVI_ROPE_GROUP(4, 4) } else if (a.nq == 3) { KIVI_ROPE_GROUP(4, 3) } else { KIVI_ROPE_GROUP(4, 2) }
        } else {
            if (a.nq == 4) { KIVI_ROPE_GROUP(2, 4) } else if (a.nq == 3) { KIVI_ROPE_GROUP(2, 3) } else { KIVI_ROPE_GROUP(2, 2) }
        }
#undef KIVI_ROPE_GROUP
        return hipGetLastError();
    }
    if (a.bits == 4) {
        if (ragged) KIVI_ROPE(4, true) else KIVI_ROPE(4, false)
    } else {
        if (ragged) KIVI_ROPE(2, true) else KIVI_ROPE(2, false)
    }
#undef KIVI_ROPE
    return hipGetLastError();
}

}  // namespace kivi
