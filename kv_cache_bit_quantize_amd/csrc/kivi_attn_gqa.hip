// kivi_attn_gqa.hip -- decode attention for grouped-query heads (gfx950).
//
// With grouped-query attention several query heads share one KV head (the query group of a
// KV head; the Mistral-7B shape has 4).  Running them one head at a time would stream the
// same 2-bit cache once per query.  Here one workgroup takes NQ query heads of a KV head and
// streams that KV head's cache once, and the query group is the M dimension of both matrix
// contractions:
//
//  * keys: the A operand of v_mfma_i32_16x16x64_i8 holds, in row 4h + d, digit d of the
//    fixed-point q_h*s (the 30-bit integer scheme of the single-query kernel), so one
//    instruction gives the four digit sums of NQ queries for 16 tokens.  Tile t (tokens
//    16t..16t+15 of the wave-iteration's 64) has its own accumulator; lane 16h + n ends
//    with query h's digit sums for token 16t + n.
//  * values: the A operand of v_mfma_f32_16x16x32_f16 holds query h's fp16 token weights
//    p*s in row h, against the same code operands as the single-query kernel, so the
//    accumulator rows are the NQ queries' outputs.
//
// Split-K, the residual, the per-query online softmax (log2 domain) and the merge follow
// the single-query kernel (kivi_attn.hip, kivi_attn_common.h).
#include <hip/hip_ext.h>

#include "kivi_attn_common.h"

namespace kivi {

template <int NQ>
struct GqaLds {
    static constexpr int kKeyGroup = NQ * 4 * kD;      // digit planes of one group: [query][digit][128 B]
    static constexpr int kWtOff = 2 * kKeyGroup;        // weights [group][chgroup][query][kg][8] fp16
    static constexpr int kWtGroup = 4 * NQ * 64;
    static constexpr int kPairOff = kWtOff + 2 * kWtGroup;   // value pairs of the 64 tokens, [64][16 B]
    static constexpr int kBytes = kPairOff + 64 * 16;
    static constexpr int kZeroBytes = kKeyGroup + 256;  // covers every offset a zero row reads at
};

// Four waves per workgroup (six and eight, at two workgroups per compute unit, measured
// slower or no faster).
constexpr int kGqaWaves = 4;
constexpr int kGqaBlock = 64 * kGqaWaves;

template <int NQ, int GS, bool RAGGED>
__global__ __launch_bounds__(kGqaBlock) __attribute__((amdgpu_waves_per_eu(3))) void attn_gqa_kernel(AttnArgs a) {
    using Lds = GqaLds<NQ>;
    constexpr int W = kGqaWaves, S = 2 * kGqaWaves;
    __shared__ __align__(16) uint8_t sh_area[W][Lds::kBytes];
    __shared__ __align__(16) uint8_t sh_zero[Lds::kZeroBytes];
    __shared__ __align__(16) float sh_o[NQ][S][kD];
    __shared__ float sh_m[NQ][S], sh_l[NQ][S];

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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, as the compiler sees it
    const int gh = lane >> 5, tt = lane & 31;        // token role (loads): token tt of group gh
    const int wl = lane & 31, wk = wl & 3;           // fixed-point writer role: channels 4wl..4wl+3
    const int mrow = lane & 15, kgrp = lane >> 4;    // matrix-operand role
    const int qh = lane >> 4, n = lane & 15;         // logit / weight role: query qh, token n of each tile
    const bool qlive = qh < NQ;
    uint8_t* area = &sh_area[wave][0];

    for (int i = threadIdx.x; i < Lds::kZeroBytes / 16; i += kGqaBlock)
        reinterpret_cast<uint4*>(sh_zero)[i] = make_uint4(0, 0, 0, 0);

    // query channels 4wl..4wl+3 of the NQ queries as packed fp16 pairs (4wl, 4wl+1 and
    // 4wl+2, 4wl+3)
    uint32_t qp[NQ][2];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        const uint2 x = *reinterpret_cast<const uint2*>(a.q + (qrow0 + r) * kD + 4 * wl);
        qp[r][0] = x.x;
        qp[r][1] = x.y;
    }
    // the largest |q| of the NQ queries per channel, times |sm_scale * log2 e|: bounds
    // |q_r * s| in the log2 domain without the products
    float qa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qa[i] = 0.0f;
#pragma unroll
        for (int r = 0; r < NQ; ++r) qa[i] = fmaxf(qa[i], fabsf(h2f(qp[r][i >> 1] >> (16 * (i & 1)))));
        qa[i] *= fabsf(a.sm_log2);
    }
    // codes of channels 4i..4i+3 arrive multiplied by 1, 4, 16, 16 (i = 0..3)
    const float cls_div = wk == 0 ? 1.0f : (wk == 1 ? 0.25f : 0.0625f);
    const float csl = cls_div * a.sm_log2;
    // a zero the compiler cannot see: fma(h, f, kZero) stays one mixed-precision fma (a
    // literal zero would turn it into a multiply with a separate conversion)
    const float kZero = __builtin_bit_cast(float, in_vgpr(0u));
    // after half_sum4, lane (r >> 1) | ((r & 1) << 1) of a half-wave holds query r's sum: the
    // byte address of this lane's query's sum in the first half (a query past NQ reads a sum
    // of zeros; its logits are -inf anyway)
    const int zsrc = 4 * ((qh >> 1) | ((qh & 1) << 1));

    // key A operand of group g, channel half kh: row 4h + d = digit plane (h, d) of the group
    // (rows of absent queries read zeros) at kbase + g*kKeyGroup + 64*kh
    const uint8_t* kbase = ((mrow >> 2) < NQ) ? area + ((mrow >> 2) * 4 + (mrow & 3)) * kD + 16 * kgrp
                                              : sh_zero + 16 * kgrp;
    // value A operand of (group g, channel group k): row h = query h's weights, at
    // vbase + (g*4 + k)*NQ*64
    const uint8_t* vbase = (mrow < NQ) ? area + Lds::kWtOff + mrow * 64 + 16 * kgrp : sh_zero + 16 * kgrp;
    // this lane's weight slots: token 16t + n of the wave-iteration is token 16(t&1) + n of
    // group t>>1; tokens 8kg..8kg+7 of a group are ordered 0,4,1,5,2,6,3,7 in their slots
    uint8_t* wbase = area + Lds::kWtOff + qh * 64 + (n >> 3) * 16 + (((n & 3) << 1) | ((n >> 2) & 1)) * 2;
    // token 4a + i meets its code as the fp16 subnormal c * 4^i * 2^-24; its weight carries
    // 16 * 4^-i, so every product is 2^-20 * (weight without the factor) * c
    const float cls_w = __builtin_ldexpf(16.0f, -2 * (n & 3));

    v4f cv[8];                          // P.V accumulators, row h = query h
#pragma unroll
    for (int v = 0; v < 8; ++v) cv[v] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    float zk[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // this lane's share (query qh) of sum p*zero, per channel group
    float lsum = 0.0f, m = -INFINITY;          // query qh's running sum and max
    float vs = 0.0f;                    // power-of-two factor keeping the value weights in fp16 range

    const RowState rs = RAGGED ? wi.rs : row_state(a);
    const int n_groups = rs.n_quant / kG;
    const int g_lo = split * rs.groups_per_split;
    const int g_hi = min(n_groups, g_lo + rs.groups_per_split);
    const int cnt = max(0, g_hi - g_lo);
    const int per_wave = (cnt + W - 1) / W;
    const int gb = g_lo + min(cnt, wave * per_wave);
    const int ge = g_lo + min(cnt, (wave + 1) * per_wave);
    const int iters = (ge - gb + 1) >> 1;

    const int64_t tok_base = kvrow * (int64_t)a.token_cap;
    const uint8_t* kc_row = a.k_codes + tok_base * kRowBytes;
    const uint8_t* vc_row = a.v_codes + tok_base * kRowBytes;
    const uint32_t* kp_row = reinterpret_cast<const uint32_t*>(a.k_sz) + kvrow * (int64_t)(a.token_cap / GS) * kD;
    const uint32_t* vp_row = reinterpret_cast<const uint32_t*>(a.v_sz) + tok_base * (kD / GS);

    constexpr uint32_t kF0 = 0x00030003u, kF1 = 0x000C000Cu, kF2 = 0x00300030u, kF3 = 0x00C000C0u;

    struct Loads {
        uint4 kp;          // (scale, zero) of key channels 4wl..4wl+3 of group gh
        uint4 kc[2];       // key tile chunk `lane` of both groups (matrix operand B)
        uint4 vc[2];       // value tile chunk `lane` of both groups (matrix operand B)
        uint4 vp;          // (scale, zero) of the 4 channel groups of token tt of group gh
    };
    // Each stream has one register set and reloads the next iteration's data right after its
    // last use in this one, so every load still has most of an iteration to arrive.
    auto group_of = [&](int it, int half) {
        const int g0 = gb + 2 * it;
        return half == 0 ? g0 : (g0 + 1 < ge ? g0 + 1 : gb);   // in-bounds address for an idle half
    };
    // uniform batches stream the cache with non-temporal loads (1-2% faster on gqa-mistral-7b);
    // the ragged batch measured 2% slower with them and keeps plain loads
    auto ld16 = [](const void* p) { return RAGGED ? *reinterpret_cast<const uint4*>(p) : stream_load16(p); };
    auto load_kp = [&](Loads& L, int it) {
        L.kp = ld16(kp_row + (int64_t)(group_of(it, gh) / (GS / kG)) * kD + 4 * wl);
    };
    auto load_kc = [&](Loads& L, int it) {
        L.kc[0] = ld16(reinterpret_cast<const uint4*>(kc_row + (int64_t)group_of(it, 0) * kTileBytes) + lane);
        L.kc[1] = ld16(reinterpret_cast<const uint4*>(kc_row + (int64_t)group_of(it, 1) * kTileBytes) + lane);
    };
    auto load_vc = [&](Loads& L, int it) {
        L.vc[0] = ld16(reinterpret_cast<const uint4*>(vc_row + (int64_t)group_of(it, 0) * kTileBytes) + lane);
        L.vc[1] = ld16(reinterpret_cast<const uint4*>(vc_row + (int64_t)group_of(it, 1) * kTileBytes) + lane);
    };
    auto load_vp = [&](Loads& L, int it) {
        L.vp = load_value_pairs<GS, !RAGGED>(vp_row + value_pair_index<GS>((int64_t)group_of(it, gh) * kG + tt, 0));
    };

    __syncthreads();   // the zero area is written
    // One register set of loads: each stream reloads it for the next iteration right after its
    // last use in this one, so every load has most of an iteration to arrive.  (Two sets, two
    // iterations ahead, with the loop body unrolled twice over them, took 168 VGPRs and ran
    // 92.6 us against 86.2 us for this form at the gqa-mistral-7b shape: the two waves per
    // SIMD that a 512-workgroup batch leaves are held by their vector work, not by latency.)
    constexpr int kPrefetch = 1;
    auto load_all = [&](Loads& L, int it) {
        load_kp(L, it);
        load_kc(L, it);
        load_vp(L, it);
        load_vc(L, it);
    };
    auto iteration = [&](Loads& cur, int it) {
        const int nxt = min(it + kPrefetch, iters - 1);
        const bool gv0 = gb + 2 * it < ge, gv1 = gb + 2 * it + 1 < ge;

        // ---- q_r*s of this half's group as 30-bit fixed point (one exponent for the NQ
        // queries), four signed byte digits per channel, stored as digit planes; q_r.z as
        // packed dot products
        float az;    // after the reduction: q_r.z of the half's group, in the lane zsrc names for r
        int sh;
        {
            const uint32_t pr[4] = {cur.kp.x, cur.kp.y, cur.kp.z, cur.kp.w};
            float s4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] = h2f(pr[i] & 0xffffu);
            // the packed queries stay packed: converting them once, outside the loop, would
            // hold 4*NQ more registers for a saving of no instruction (the conversions fold
            // into the mixed-precision products)
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                asm volatile("" : "+v"(qp[r][0]));
                asm volatile("" : "+v"(qp[r][1]));
            }
            float mx = fmaxf(fmaxf(qa[0] * s4[0], qa[1] * s4[1]), fmaxf(qa[2] * s4[2], qa[3] * s4[3]));
            const uint32_t z01 = __builtin_amdgcn_perm(pr[1], pr[0], 0x07060302u);   // zeros of 4wl, 4wl+1
            const uint32_t z23 = __builtin_amdgcn_perm(pr[3], pr[2], 0x07060302u);
            float az4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < NQ; ++r)
                az4[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qp[r][0]), __builtin_bit_cast(h2v, z01),
                                                __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qp[r][1]),
                                                                       __builtin_bit_cast(h2v, z23), 0.0f, false),
                                                false);
            az = half_sum4(az4);
            mx = half_max_nonneg(mx);
            sh = min(29 - __builtin_amdgcn_frexp_expf(mx), 100);   // |q*s| * 2^sh < 2^29
            const float ff = __builtin_ldexpf(csl, sh);
            float sf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sf[i] = s4[i] * ff;
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                uint32_t dg[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // truncated: off by less than 2^-29 of the largest
                    const int qi = (int)__builtin_fmaf(h2f(qp[r][i >> 1] >> (16 * (i & 1))), sf[i], kZero);
                    dg[i] = ((uint32_t)qi + 0x80808080u) ^ 0x80808080u;    // four signed base-256 digits
                }
                const uint32_t A = __builtin_amdgcn_perm(dg[1], dg[0], 0x05010400u);
                const uint32_t B = __builtin_amdgcn_perm(dg[1], dg[0], 0x07030602u);
                const uint32_t C = __builtin_amdgcn_perm(dg[3], dg[2], 0x05010400u);
                const uint32_t E = __builtin_amdgcn_perm(dg[3], dg[2], 0x07030602u);
                uint32_t* plane = reinterpret_cast<uint32_t*>(area + gh * Lds::kKeyGroup + r * 4 * kD) + wl;
                plane[0 * kD / 4] = __builtin_amdgcn_perm(C, A, 0x05040100u);   // digit 0 of the 4 channels
                plane[1 * kD / 4] = __builtin_amdgcn_perm(C, A, 0x07060302u);   // digit 1
                plane[2 * kD / 4] = __builtin_amdgcn_perm(E, B, 0x05040100u);   // digit 2
                plane[3 * kD / 4] = __builtin_amdgcn_perm(E, B, 0x07060302u);   // digit 3
            }
        }
        // the largest value scale among this lane's loaded token (fp16 bit patterns: scales
        // are never negative); every token's pairs are loaded by exactly one lane
        const float smax = h2f(max_u16x2(max_u16x2(cur.vp.x, cur.vp.y), max_u16x2(cur.vp.z, cur.vp.w)) & 0xffffu);
        // value pairs of the 64 tokens, for the lanes that need another lane's token
        *reinterpret_cast<uint4*>(area + Lds::kPairOff + lane * 16) = cur.vp;
        load_vp(cur, nxt);
        load_kp(cur, nxt);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- key logits: tile t = 2*group + token half, K = 64 channels per instruction;
        // each tile's digit sums are combined as soon as its two instructions are done
        float kscale[2], azq[2];   // per group: exponent and q.z of this lane's query
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            kscale[g] = __builtin_ldexpf(1.0f, -__builtin_amdgcn_readlane(sh, 32 * g));
            // one cross-lane read through the LDS crossbar (no vector-ALU selects)
            const float z = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(zsrc + 128 * g, __builtin_bit_cast(int, az)));
            azq[g] = z * a.sm_log2;
        }
        float lg[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v4i ct = {0, 0, 0, 0};
            const uint4 kc = cur.kc[t >> 1];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const uint32_t x = (t & 1) ? (kh ? kc.w : kc.z) : (kh ? kc.y : kc.x);
                const v4i bop = {(int)(x & 0x03030303u), (int)(x & 0x0C0C0C0Cu), (int)(x & 0x30303030u),
                                 (int)((x >> 2) & 0x30303030u)};
                const v4i aop = *reinterpret_cast<const v4i*>(kbase + (t >> 1) * Lds::kKeyGroup + 64 * kh);
                ct = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, ct, 0, 0, 0);
            }
            const int hi = ct[3] * 256 + ct[2], lo = ct[1] * 256 + ct[0];
            const float tot = fmaf((float)hi, 65536.0f, (float)lo);
            const bool ok = qlive && ((t >> 1) ? gv1 : gv0);
            lg[t] = ok ? fmaf(tot, kscale[t >> 1], azq[t >> 1]) : -INFINITY;
        }
        load_kc(cur, nxt);

        // ---- online softmax per query over the 64 tokens (rescale only when a max rises)
        const float mnew = fmax_ieee(m, row_max(fmax_ieee(fmax_ieee(lg[0], lg[1]), fmax_ieee(lg[2], lg[3]))));
        const float al = mnew == m ? 1.0f : exp2_fast(m - mnew);
        if (__builtin_amdgcn_ballot_w64(al < 1.0f)) {
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                const float ar = readlane_f(al, 16 * r);
#pragma unroll
                for (int v = 0; v < 8; ++v) cv[v][r] *= ar;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) zk[k] *= al;
            lsum *= al;
        }
        m = mnew;
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            p[t] = lg[t] == -INFINITY ? 0.0f : exp2_fast(lg[t] - m);
            lsum += p[t];
        }
        // value pairs of this lane's 4 tokens 16t + n: zero-point sums
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 pq = *reinterpret_cast<const uint4*>(area + Lds::kPairOff + (16 * t + n) * 16);
            const uint32_t pw[4] = {pq.x, pq.y, pq.z, pq.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) zk[k] = fmaf(p[t], h2f(pw[k] >> 16), zk[k]);
        }
        // value weights 16*p*s*vs must stay below 2^15: shrink vs (a power of two) if needed
        if (__builtin_amdgcn_ballot_w64(smax * vs > 2048.0f || vs == 0.0f)) {
            const float gm = wave_max_xor(smax, 1, 32);
            const float nvs = __builtin_ldexpf(1.0f, 11 - __builtin_amdgcn_frexp_expf(gm));
            if (vs != 0.0f && nvs < vs) {
                const float rs = nvs / vs;
#pragma unroll
                for (int v = 0; v < 8; ++v) cv[v] *= rs;
            }
            if (vs == 0.0f || nvs < vs) vs = nvs;
        }
        if (qlive) {   // the weights, from the pairs read again
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 pq = *reinterpret_cast<const uint4*>(area + Lds::kPairOff + (16 * t + n) * 16);
                const uint32_t pw[4] = {pq.x, pq.y, pq.z, pq.w};
                const float f = p[t] * (cls_w * vs);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    *reinterpret_cast<_Float16*>(wbase + (t >> 1) * Lds::kWtGroup + (t & 1) * 32 + k * NQ * 64) =
                        (_Float16)(f * h2f(pw[k] & 0xffffu));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- P.V: K = the 32 tokens of a group, N = 16 channels, M = the NQ queries
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint4 vc = cur.vc[g];
            const uint32_t words[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                // token field i of each byte, masked in place: the fp16 subnormal c * 4^i * 2^-24
                const uint32_t x = (v & 1) ? words[v >> 1] >> 8 : words[v >> 1];
                const v8h bop = __builtin_bit_cast(v8h, make_uint4(x & kF0, x & kF1, x & kF2, x & kF3));
                const v8h aop = *reinterpret_cast<const v8h*>(vbase + (g * 4 + (v >> 1)) * NQ * 64);
                cv[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, cv[v], 0, 0, 0);
            }
        }
        load_vc(cur, nxt);
    };
    // Every load is issued unconditionally (past the end it reads the last iteration's data
    // again, from the L2) and the loop has one exit, at its head, so both paths into the head
    // have issued the same loads: the compiler then knows how many loads are in flight at
    // each use and waits for exactly the one it needs.  When a wave's range has an odd number
    // of groups, its last iteration's second half is idle: that group is out of range, so its
    // logits are -inf and its weights zero.
    Loads set0;
    uint32_t tag;
    if (iters > 0) {
        load_all(set0, 0);
        tag = settle_tag(tag_v);
        // The SIMDs issue the oldest waves first, so of a CU's workgroups the first launched
        // runs ahead and the last finishes alone, with too few waves to hide its loads.  Each
        // wave instead takes a priority from the iterations it has left (most left, highest),
        // so the waves sharing a SIMD draw level and finish together.
        for (int it = 0; it < iters; ++it) {
            set_priority_for(iters - it);
            iteration(set0, it);
        }
        __builtin_amdgcn_s_setprio(0);
    } else {
        tag = settle_tag(tag_v);
    }

    // ---- each query's quantized-part state: o = P.V * 2^20 / vs + sum p*zero
    lsum = row_sum(lsum);
#pragma unroll
    for (int k = 0; k < 4; ++k) zk[k] = row_sum(zk[k]);
    const float inv = vs != 0.0f ? 1048576.0f / vs : 0.0f;
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        float zr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) zr[k] = readlane_f(zk[k], 16 * r);
        if (lane < 16) {   // accumulator row r: channel 16v + lane
#pragma unroll
            for (int v = 0; v < 8; ++v) sh_o[r][wave][16 * v + lane] = fmaf(cv[v][r], inv, zr[v >> 1]);
        }
        const float mq = readlane_f(m, 16 * r), lq = readlane_f(lsum, 16 * r);
        if (lane == 0) {
            sh_m[r][wave] = mq;
            sh_l[r][wave] = lq;
        }
    }

    // ---- fp16 residual (last split only), as separate states.  The scheduling barrier keeps
    // its loads from being hoisted above this point, where the accumulators are still live.
    __builtin_amdgcn_sched_barrier(0);
    float mr[NQ], lr[NQ];
    if (split == rs.res_split) {
        __builtin_amdgcn_s_setprio(2);   // the residual is work the other splits do not have
        residual_states<NQ, W>(a, rs, qrow0, kvrow, wave, &sh_o[0][W + wave][0], S * kD, mr, lr);
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
            sh_m[r][W + wave] = mr[r];
            sh_l[r][W + wave] = lr[r];
        }
    }
    __syncthreads();
    finish_block<NQ, W>(a, rs.splits, split, qrow0, tag, sh_o, sh_m, sh_l);
}

hipError_t launch_decode_attn_gqa(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid = attn_grid(a, a.block_rows);
#define KIVI_GQA_NQ(NQv)                                                                                          \
    if (a.seq_state != nullptr)                                                                                   \
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_gqa_kernel<NQv, GS, true>), grid, dim3(kGqaBlock), 0, s, \
                                                     t0, t1, 0, a))                                               \
    else                                                                                                          \
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_gqa_kernel<NQv, GS, false>), grid, dim3(kGqaBlock), 0, s, \
                                                     t0, t1, 0, a))
    switch (a.nq) {
        case 2: KIVI_GQA_NQ(2) break;
        case 3: KIVI_GQA_NQ(3) break;
        case 4: KIVI_GQA_NQ(4) break;
        default: return hipErrorInvalidValue;
    }
#undef KIVI_GQA_NQ
    return hipGetLastError();
}

}  // namespace kivi
