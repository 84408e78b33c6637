// kivi_attn.hip -- fused decode attention over the 2-bit cache (gfx950).
//
// One query per head attends over the dequantized history followed by the fp16
// residual: out = softmax(sm_scale * q.K^T) . V (error judged at the attention output:
// article "Your KV cache doesn't have a bit problem...", paragraph 3).
//
// Work split: grid (splits, B*Hq), sized for one workgroup per CU.  A 12-wave workgroup owns
// one query row and a contiguous range of key groups, taken two groups (64 tokens) at a time
// by its waves from an LDS counter, each wave with its own online softmax (log2 domain).  A
// CU favours its oldest waves when it issues; with one workgroup per CU and the pairs handed
// out on demand, all of the CU's waves still finish together (with three 4-wave workgroups
// per CU and fixed quarters, the youngest workgroup ended about 10% after the oldest).  The
// split holding the last groups first reads the fp16 residual, as separate softmax states,
// and its waves join the queue after it.  The workgroup merges its states in LDS and writes
// one partial (o[128], m, l); the last workgroup of the row to arrive merges the row's
// partials with the log-sum-exp merge and writes the output, so one launch does the whole
// call.
//
// Inner loop: one wave-iteration = two 32-token groups (64 tokens).  The 2-bit codes make
// the loop bound by HBM and by the instructions that turn codes into products, so both
// contractions run on the matrix cores and the vector units only prepare operands:
//
//  * keys, per token group g: q.(z + c*s) = q.z + (q*s).c.  The 32 lanes of a half-wave
//    compute q*s for 4 channels each, turn it into a 30-bit fixed-point integer with a
//    per-group exponent and split it into four signed byte digits, stored in LDS as four
//    128-byte digit planes.  v_mfma_i32_16x16x64_i8 then multiplies those digits (A,
//    rows = digits) with the codes (B, one token per column; a code word masked with
//    0x03030303 << 2i gives channels 4i..4i+3 as bytes, the factor 4^i divided out of
//    the fixed-point values beforehand).  The products are exact integers.  Tile t (16
//    tokens) puts its digits in rows 4t..4t+3 and zeros elsewhere, so one accumulator
//    leaves lane L with the four digit sums of token L.
//  * values, per token: p*(z + c*s) = p*z + (p*s)*c.  Each lane's token weight p*s is
//    rounded to fp16 and stored in LDS in the A-operand order of v_mfma_f32_16x16x32_f16
//    (row 0; the other rows read zeros).  The codes become B operands by masking in place:
//    token field i of a code byte under the mask 0x00030003 << 2i (the odd 16-channel
//    blocks after one shift by 8) is the fp16 subnormal c * 4^i * 2^-24, which the matrix
//    cores multiply exactly.  The weight carries 16 * 4^-i and a power of two vs keeping it
//    in fp16 range, so every product is 2^-20 * vs * p*s*c, and o = C * 2^20 / vs + sum p*z
//    with the zero-point part sum p*z accumulated on the vector units.
#include <hip/hip_ext.h>

#include "kivi_attn_common.h"

namespace kivi {

// LDS area of one (parity, wave)
constexpr int kGroupTbl = 4 * kD;                 // key digit planes of one group: 4 x 128 B
constexpr int kWtOff = 2 * kGroupTbl;             // value weights [group][chgroup][kg][8] fp16
constexpr int kZeroOff = kWtOff + 2 * 4 * 4 * 16;  // 512 zero bytes
constexpr int kAreaBytes = kZeroOff + 512;

// W: waves per workgroup.  12 (one workgroup per CU) when the call has few rows and splits
// them; 4 (three workgroups per CU) when a uniform batch has more query rows than the chip has
// CUs, so that its rows run in one round of resident workgroups instead of several rounds that
// each pay the start-up again.
template <int GS, int W, bool RAGGED>
__global__ __launch_bounds__(64 * W) void attn_split_kernel(AttnArgs a) {
    constexpr int kSqWaves = W, kSqSlots = 2 * W;
    __shared__ __align__(16) uint8_t sh_area[2][kSqWaves][kAreaBytes];
    __shared__ __align__(16) float sh_o[1][kSqSlots][kD];
    __shared__ float sh_m[1][kSqSlots], sh_l[1][kSqSlots];
    __shared__ int sh_next;   // pair queue of the workgroup's range (pairs past the static ones)

    // (ragged batch: the plan uses sh_o, unused until the end)
    const WorkItem wi = work_item<RAGGED>(a, reinterpret_cast<int32_t*>(&sh_o[0][0][0]));
    if (RAGGED && wi.split < 0) return;   // (ragged batch) past the plan's last item
    const int split = wi.split;
    const int64_t qrow = wi.row;
    // Query row b*Hq + h reads kv row b*Hkv + h/ratio = qrow/ratio (Hq = Hkv*ratio): one 32-bit
    // division, none for one query per kv head.  The set-up before the first loads is kept short:
    // each of its instructions delays them, and a CU issues it for three waves per SIMD.
    const int64_t kvrow = a.ratio == 1 ? qrow : (int64_t)((uint32_t)qrow / (uint32_t)a.ratio);
    if (a.k_new != nullptr && split == 0 && (uint32_t)qrow % (uint32_t)a.ratio == 0) store_new_token(a, kvrow);
    const TagLoads<1> tag_v = partial_tag<1>(a, qrow);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, as the compiler sees it
    const int gh = lane >> 5;          // group of the wave-iteration this lane serves
    const int tt = lane & 31;          // token role: token tt of group gh
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

    // Key A operand of tile t: rows 4t..4t+3 hold digits 0..3 of the tile's group, all
    // other rows are zero; this lane's 16 bytes come from its digit plane or the zeros.
    int ka_off[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        ka_off[t] = ((mrow >> 2) == t) ? (t >> 1) * kGroupTbl + (mrow & 3) * kD + 16 * kgrp : kZeroOff + 16 * kgrp;
    // Value A operand of (group, channel group): row 0 holds the weights, other rows zero.
    const int va_off = (mrow == 0 ? kWtOff : kZeroOff) + 16 * kgrp;
    // this lane's slot in the weight table: tokens 8kg..8kg+7 of a group are ordered
    // 0,4,1,5,2,6,3,7 (the order the code operand produces them in)
    const int w_off = kWtOff + gh * 4 * 64 + (tt >> 3) * 16 + (((tt & 3) << 1) | ((tt >> 2) & 1)) * 2;
    // token 4a + i meets its code as the fp16 subnormal c * 4^i * 2^-24; its weight carries
    // 16 * 4^-i, so every product is 2^-20 * (weight without the factor) * c
    const float cls_w = __builtin_ldexpf(16.0f, -2 * (tt & 3));
    // the zero areas of both parities, written once
    reinterpret_cast<uint4*>(&sh_area[lane >> 5][wave][kZeroOff])[lane & 31] = make_uint4(0, 0, 0, 0);

    v4f cv[8];                         // P.V accumulators, one per 16-channel block (row 0)
#pragma unroll
    for (int v = 0; v < 8; ++v) cv[v] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    float zk[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // ... and of sum p*zero, per channel group
    float lsum = 0.0f, m = -INFINITY;
    float vs = 0.0f;                   // power-of-two factor keeping the value weights in fp16 range

    const RowState rs = RAGGED ? wi.rs : row_state(a);
    const int n_groups = rs.n_quant / kG;
    const int g_lo = split * rs.groups_per_split;
    const int g_hi = min(n_groups, g_lo + rs.groups_per_split);
    const int n_pairs = (max(0, g_hi - g_lo) + 1) >> 1;   // the workgroup's pairs of 32-token tiles
    // Pair schedule: wave w takes pairs w and w + kSqWaves, then one pair per iteration from
    // the workgroup's LDS counter, requested one iteration before it is needed.  Pairs are
    // handed out in increasing order, so a wave stops at its first pair past the range and
    // no pair is skipped.  The waves of a CU's workgroup thereby finish together however the
    // CU's issue arbitration favours them.
    int c_cur = wave, c_nxt = wave + kSqWaves, pend = 0;

    const int64_t tok_base = kvrow * (int64_t)a.token_cap;
    const uint8_t* kc_row = a.k_codes + tok_base * kRowBytes;
    const uint8_t* vc_row = a.v_codes + tok_base * kRowBytes;
    const uint32_t* kp_row = reinterpret_cast<const uint32_t*>(a.k_sz) + kvrow * (int64_t)(a.token_cap / GS) * kD;
    const uint32_t* vp_row = reinterpret_cast<const uint32_t*>(a.v_sz) + tok_base * (kD / GS);

    constexpr uint32_t kF0 = 0x00030003u, kF1 = 0x000C000Cu, kF2 = 0x00300030u, kF3 = 0x00C000C0u;

    // one wave-iteration's global loads (issued one iteration ahead of their use); every
    // load instruction reads a contiguous span
    struct Loads {
        uint4 kp;          // (scale, zero) of key channels 4wl..4wl+3 of group gh
        uint4 kc[2];       // key tile chunk `lane` of both groups (matrix operand B)
        uint4 vc[2];       // value tile chunk `lane` of both groups (matrix operand B)
        uint4 vp;          // (scale, zero) of the 4 channel groups of token tt of group gh
    };
    // Each stream has one register set and reloads the next iteration's data right after its
    // last use in this one, so every load still has most of an iteration to arrive.
    // first groups of the current and the next iteration (wave-uniform)
    int g_cur0 = g_lo + 2 * c_cur;
    int g_nxt0 = c_nxt < n_pairs ? g_lo + 2 * c_nxt : 0;
    auto group_of = [&](int which, int half) {   // which: 0 = current iteration, 1 = next
        const int g0 = which ? g_nxt0 : g_cur0;
        return half == 0 ? g0 : (g0 + 1 < g_hi ? g0 + 1 : g0);   // in-bounds address for an idle half
    };
    // the cache streams through with non-temporal loads: 403 MB at the 131,072-token context in
    // 64.1-64.4 us against 72.4-72.6 us with plain loads (same GPU, same outputs)
    auto load_kp = [&](Loads& L, int it) {
        L.kp = stream_load16(kp_row + (int64_t)(group_of(it, gh) / (GS / kG)) * kD + 4 * wl);
    };
    auto load_kc = [&](Loads& L, int it) {
        L.kc[0] = stream_load16(reinterpret_cast<const uint4*>(kc_row + (int64_t)group_of(it, 0) * kTileBytes) + lane);
        L.kc[1] = stream_load16(reinterpret_cast<const uint4*>(kc_row + (int64_t)group_of(it, 1) * kTileBytes) + lane);
    };
    auto load_vc = [&](Loads& L, int it) {
        L.vc[0] = stream_load16(reinterpret_cast<const uint4*>(vc_row + (int64_t)group_of(it, 0) * kTileBytes) + lane);
        L.vc[1] = stream_load16(reinterpret_cast<const uint4*>(vc_row + (int64_t)group_of(it, 1) * kTileBytes) + lane);
    };
    auto load_vp = [&](Loads& L, int it) {
        L.vp = load_value_pairs<GS, true>(vp_row + value_pair_index<GS>((int64_t)group_of(it, gh) * kG + tt, 0));
    };

    // Every load is issued unconditionally, so the compiler knows how many loads are in flight
    // at each use and waits for exactly the one it needs.  Past the end a wave reads the row's
    // first two groups: the row's 96 waves share those lines, so they mostly come from the L2
    // (re-reading the wave's own last pair, which the non-temporal loads do not keep, cost
    // 3.7% more HBM bytes and about 1 us at the 131,072-token context).
    Loads cur;
    if (c_cur < n_pairs) {   // the first iteration's loads, in flight during the set-up below
        load_kp(cur, 0);
        load_kc(cur, 0);
        load_vp(cur, 0);
        load_vc(cur, 0);
    }
    if (threadIdx.x == 0) sh_next = 0;
    __syncthreads();

    // ---- fp16 residual first (split rs.res_split), as separate states: its loads meet a memory
    // system that is not loaded yet, and the waves that take it start on the pairs later
    float mr[1] = {-INFINITY}, lr[1] = {0.0f};
    if (split == rs.res_split)
        residual_states<1, kSqWaves>(a, rs, qrow, kvrow, wave, &sh_o[0][kSqWaves + wave][0], kSqSlots * kD, mr, lr);
    if (c_cur < n_pairs && lane == 0) pend = atomicAdd(&sh_next, 1);

    uint32_t tag;
    if (c_cur < n_pairs) {
        tag = settle_tag(tag_v);
        for (int it = 0;;) {
            constexpr int nxt = 1;
            const bool gvalid = g_cur0 + gh < g_hi;
            uint8_t* area = &sh_area[it & 1][wave][0];

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
            mx = half_max_nonneg(mx);
            const int sh = min(29 - __builtin_amdgcn_frexp_expf(mx), 100);   // |q*s| * 2^sh < 2^29
            const float fs = __builtin_ldexpf(cls_div, sh);
            uint32_t dg[4];
    #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int qi = (int)(qs[i] * fs);   // truncated: off by less than 2^-29 of the largest
                dg[i] = ((uint32_t)qi + 0x80808080u) ^ 0x80808080u;    // four signed base-256 digits
            }
            {
                const uint32_t A = __builtin_amdgcn_perm(dg[1], dg[0], 0x05010400u);
                const uint32_t B = __builtin_amdgcn_perm(dg[1], dg[0], 0x07030602u);
                const uint32_t C = __builtin_amdgcn_perm(dg[3], dg[2], 0x05010400u);
                const uint32_t E = __builtin_amdgcn_perm(dg[3], dg[2], 0x07030602u);
                uint32_t* plane = reinterpret_cast<uint32_t*>(area + gh * kGroupTbl) + wl;
                plane[0 * kD / 4] = __builtin_amdgcn_perm(C, A, 0x05040100u);   // digit 0 of the 4 channels
                plane[1 * kD / 4] = __builtin_amdgcn_perm(C, A, 0x07060302u);   // digit 1
                plane[2 * kD / 4] = __builtin_amdgcn_perm(E, B, 0x05040100u);   // digit 2
                plane[3 * kD / 4] = __builtin_amdgcn_perm(E, B, 0x07060302u);   // digit 3
            }
            load_kp(cur, nxt);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // ---- key logits on the matrix cores: tile t = 2*group + token half, K = 64
            // channels per instruction
            v4i cacc = {0, 0, 0, 0};
    #pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 kc = cur.kc[t >> 1];
    #pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    const uint32_t x = (t & 1) ? (kh ? kc.w : kc.z) : (kh ? kc.y : kc.x);
                    const v4i bop = {(int)(x & 0x03030303u), (int)(x & 0x0C0C0C0Cu), (int)(x & 0x30303030u),
                                     (int)((x >> 2) & 0x30303030u)};
                    const v4i aop = *reinterpret_cast<const v4i*>(area + ka_off[t] + 64 * kh);
                    cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop, cacc, 0, 0, 0);
                }
            }
            load_kc(cur, nxt);
            float lg;
            {
                const int hi = cacc[3] * 256 + cacc[2], lo = cacc[1] * 256 + cacc[0];
                const float tot = fmaf((float)hi, 65536.0f, (float)lo);
                lg = gvalid ? fmaf(tot, __builtin_ldexpf(1.0f, -sh), az) : -INFINITY;
            }

            // ---- online softmax over the wave's 64 tokens (rescale only when the max rises)
            float mloc = half_max(lg);
            mloc = fmax_ieee(readlane_f(mloc, 0), readlane_f(mloc, 32));
            if (mloc > m) {
                const float al = exp2_fast(m - mloc);
    #pragma unroll
                for (int v = 0; v < 8; ++v) cv[v] *= al;
    #pragma unroll
                for (int k = 0; k < 4; ++k) zk[k] *= al;
                lsum *= al;
                m = mloc;
            }
            const float p = exp2_fast(lg - m);   // this lane's token
            lsum += p;
            const uint32_t vpr[4] = {cur.vp.x, cur.vp.y, cur.vp.z, cur.vp.w};
    #pragma unroll
            for (int k = 0; k < 4; ++k) zk[k] = fmaf(p, h2f(vpr[k] >> 16), zk[k]);
            // the largest scale, on the fp16 bit patterns (scales are never negative)
            const float smax = h2f(max_u16x2(max_u16x2(vpr[0], vpr[1]), max_u16x2(vpr[2], vpr[3])) & 0xffffu);
            // value weights 16*p*s*vs must stay below 2^15: shrink vs (a power of two) if needed
            if (__builtin_amdgcn_ballot_w64(smax * vs > 2048.0f || vs == 0.0f)) {
                const float gm = wave_max_xor(smax, 1, 32);
                const float nvs = __builtin_ldexpf(1.0f, 11 - __builtin_amdgcn_frexp_expf(gm));
                if (vs != 0.0f && nvs < vs) {
                    const float r = nvs / vs;
    #pragma unroll
                    for (int v = 0; v < 8; ++v) cv[v] *= r;
                }
                if (vs == 0.0f || nvs < vs) vs = nvs;
            }
            {
                const float f = p * (cls_w * vs);
    #pragma unroll
                for (int k = 0; k < 4; ++k)
                    *reinterpret_cast<_Float16*>(area + w_off + k * 64) = (_Float16)(f * h2f(vpr[k] & 0xffffu));
            }
            load_vp(cur, nxt);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // ---- P.V on the matrix cores: K = the 32 tokens of a group, N = 16 channels
    #pragma unroll
            for (int g = 0; g < 2; ++g) {
                const uint4 vc = cur.vc[g];
                const uint32_t words[4] = {vc.x, vc.y, vc.z, vc.w};
    #pragma unroll
                for (int v = 0; v < 8; ++v) {
                    // word v/2 holds blocks v (even) and v+1 in alternate bytes; token field i
                    // of each byte, masked in place, is the fp16 subnormal c * 4^i * 2^-24
                    const uint32_t x = (v & 1) ? words[v >> 1] >> 8 : words[v >> 1];
                    const v8h bop = __builtin_bit_cast(v8h, make_uint4(x & kF0, x & kF1, x & kF2, x & kF3));
                    const v8h aop = *reinterpret_cast<const v8h*>(area + va_off + (g * 4 + (v >> 1)) * 64);
                    cv[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, cv[v], 0, 0, 0);
                }
            }
            load_vc(cur, nxt);
            ++it;
            c_cur = c_nxt;
            if (c_cur >= n_pairs) break;
            int pv = pend;
            asm volatile("" : "+v"(pv));   // the request is read here, one iteration after it was made
            c_nxt = 2 * kSqWaves + __builtin_amdgcn_readfirstlane(pv);
            if (lane == 0) pend = atomicAdd(&sh_next, 1);
            g_cur0 = g_lo + 2 * c_cur;
            g_nxt0 = c_nxt < n_pairs ? g_lo + 2 * c_nxt : 0;
        }
    } else {
        tag = settle_tag(tag_v);
    }

    // ---- the wave's quantized-part state: o = P.V * 2^20 / vs + sum p*zero
    lsum = wave_sum(lsum);
#pragma unroll
    for (int k = 0; k < 4; ++k) zk[k] = wave_sum(zk[k]);
    if (lane < 16) {   // row 0 of the accumulators: channel 16v + lane
        const float inv = vs != 0.0f ? 1048576.0f / vs : 0.0f;
#pragma unroll
        for (int v = 0; v < 8; ++v) sh_o[0][wave][16 * v + lane] = fmaf(cv[v][0], inv, zk[v >> 1]);
    }
    if (lane == 0) {
        sh_m[0][wave] = m;
        sh_l[0][wave] = lsum;
    }

    if (lane == 0) {
        sh_m[0][kSqWaves + wave] = mr[0];
        sh_l[0][kSqWaves + wave] = lr[0];
    }
    __syncthreads();
    finish_block<1, kSqWaves>(a, rs.splits, split, qrow, tag, sh_o, sh_m, sh_l);
}

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    if (a.bits == 4) return launch_decode_attn_q4(a, s, t0, t1);
    if (a.nq > 1) return launch_decode_attn_gqa(a, s, t0, t1);
    if (a.seq_state != nullptr) {   // ragged batches: one 12-wave workgroup per CU
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_split_kernel<GS, kSqWaves, true>), attn_grid(a, a.q_rows),
                                                     dim3(64 * kSqWaves), 0, s, t0, t1, 0, a))
    } else if (a.sq_waves == 4) {
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_split_kernel<GS, 4, false>), attn_grid(a, a.q_rows),
                                                     dim3(64 * 4), 0, s, t0, t1, 0, a))
    } else {
        KIVI_BY_GROUP(a.group, hipExtLaunchKernelGGL((attn_split_kernel<GS, kSqWaves, false>), attn_grid(a, a.q_rows),
                                                     dim3(64 * kSqWaves), 0, s, t0, t1, 0, a))
    }
    return hipGetLastError();
}

}  // namespace kivi
