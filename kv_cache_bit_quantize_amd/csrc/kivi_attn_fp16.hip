// kivi_attn_fp16.hip -- decode attention over a plain fp16 KV cache (gfx950).
//
// The comparator for the 2-bit cache: the same call shape, query grouping, split-K and
// log-sum-exp merge as the quantized kernels, over keys and values held in fp16 (512 bytes
// per token and KV head, against 96 for a 2-bit token).  Decode over an fp16 cache is a
// stream of those bytes with little arithmetic per byte, so the kernel is built for the
// load stream: every load is 16 bytes per lane and coalesced, issued one iteration ahead,
// and the products run on the vector units (v_dot2_f32_f16 for q.k, mixed-precision fma
// for P.V) with fp32 accumulation.
//
// Per wave-iteration of 16 tokens:
//  * logits: lane 4t + c holds token t and channels [32c, 32c+32) (64 contiguous bytes of
//    the key row); q.k for each of the NQ query heads of the workgroup, the four channel
//    quarters summed in the quad;
//  * online softmax per query head (log2 domain), the probabilities into LDS;
//  * P.V: lane 16g + c holds tokens 4g..4g+3 and channels [8c, 8c+8) (16 lanes read one
//    256-byte value row); it accumulates its share of o for each query head, and the four
//    token groups' shares are summed once, after the loop.
#include <hip/hip_ext.h>

#include "kivi_attn_common.h"

namespace kivi {

constexpr int kF16Tok = 16;   // tokens per wave-iteration

template <int NQ>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void attn_fp16_kernel(AttnArgs a) {
    __shared__ __align__(16) float sh_p[kWaves][NQ][kF16Tok];
    __shared__ __align__(16) float sh_o[NQ][kSlots][kD];
    __shared__ float sh_m[NQ][kSlots], sh_l[NQ][kSlots];

    const int split = blockIdx.x;
    const int64_t grow = blockIdx.y;                 // (batch, kv head, query chunk)
    const int chunks = a.ratio / NQ;
    // grow = kvrow*chunks + chunk and Hq = Hkv*ratio = Hkv*chunks*NQ, so the first query row is
    // kvrow*ratio + chunk*NQ = grow*NQ: one 32-bit division (none when a kv head's query group
    // is one workgroup) before the first loads
    const int64_t kvrow = chunks == 1 ? grow : (int64_t)((uint32_t)grow / (uint32_t)chunks);
    const int64_t qrow0 = grow * NQ;
    const TagLoads<NQ> tag_v = partial_tag<NQ>(a, qrow0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kt = lane >> 2, kq = lane & 3;        // logits: token kt, channels 32kq..32kq+31
    const int vg = lane >> 4, vc = lane & 15;       // values: tokens 4vg..4vg+3, channels 8vc..8vc+7

    // this wave's tokens: a contiguous run of the split's, in whole iterations
    const int t_lo = split * a.tokens_per_split;
    const int t_hi = min(a.n_tokens, t_lo + a.tokens_per_split);
    const int cnt = max(0, t_hi - t_lo);
    const int per_wave = ((cnt + kWaves - 1) / kWaves + kF16Tok - 1) / kF16Tok * kF16Tok;
    const int tb = t_lo + min(cnt, wave * per_wave);
    const int te = t_lo + min(cnt, (wave + 1) * per_wave);
    const int iters = (te - tb + kF16Tok - 1) / kF16Tok;

    // query channels 32kq..32kq+31 of the NQ heads, packed fp16 pairs
    uint32_t qp[NQ][16];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        const uint4* src = reinterpret_cast<const uint4*>(a.q + (qrow0 + r) * kD + 32 * kq);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 x = src[i];
            qp[r][4 * i] = x.x;
            qp[r][4 * i + 1] = x.y;
            qp[r][4 * i + 2] = x.z;
            qp[r][4 * i + 3] = x.w;
        }
    }

    const uint16_t* krow = a.kf + kvrow * a.kv_stride * kD;
    const uint16_t* vrow = a.vf + kvrow * a.kv_stride * kD;
    struct Loads {
        uint4 k[4];   // key token kt, channels 32kq..32kq+31
        uint4 v[4];   // value tokens 4vg..4vg+3, channels 8vc..8vc+7
    };
    // token index clamped into the wave's range (an idle lane re-reads the first token)
    auto tok = [&](int it, int j) {
        const int t = tb + it * kF16Tok + j;
        return t < te ? t : tb;
    };
    auto load_k = [&](Loads& L, int it) {
        const uint4* p = reinterpret_cast<const uint4*>(krow + (int64_t)tok(it, kt) * kD + 32 * kq);
#pragma unroll
        for (int i = 0; i < 4; ++i) L.k[i] = p[i];
    };
    auto load_v = [&](Loads& L, int it) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            L.v[u] = *reinterpret_cast<const uint4*>(vrow + (int64_t)tok(it, 4 * vg + u) * kD + 8 * vc);
    };

    float m[NQ], lsum[NQ], o[NQ][8];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        m[r] = -INFINITY;
        lsum[r] = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[r][c] = 0.0f;
    }
    float* pw = &sh_p[wave][0][0];

    // One register set per stream, reloaded for the next iteration right after its last
    // use; every load is issued unconditionally (clamped past the end), so the compiler
    // counts the loads in flight exactly.
    Loads cur;
    uint32_t tag;
    if (iters > 0) {
        load_k(cur, 0);
        load_v(cur, 0);
        tag = settle_tag(tag_v);
        for (int it = 0; it < iters; ++it) {
            const int nxt = min(it + 1, iters - 1);
            const bool valid = tb + it * kF16Tok + kt < te;
            float lg[NQ];
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                float d = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t w[4] = {cur.k[i].x, cur.k[i].y, cur.k[i].z, cur.k[i].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qp[r][4 * i + j]), __builtin_bit_cast(h2v, w[j]),
                                                   d, false);
                }
                lg[r] = valid ? quad_sum(d) * a.sm_log2 : -INFINITY;
            }
            load_k(cur, nxt);

            // online softmax per query head over the 16 tokens
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                const float mnew = fmaxf(m[r], wave_max_quads(lg[r]));   // finite: every iteration has a token
                if (mnew != m[r]) {
                    const float al = m[r] == -INFINITY ? 0.0f : exp2f(m[r] - mnew);
#pragma unroll
                    for (int c = 0; c < 8; ++c) o[r][c] *= al;
                    lsum[r] *= al;
                    m[r] = mnew;
                }
                const float p = valid ? exp2f(lg[r] - m[r]) : 0.0f;
                lsum[r] += p;   // every lane of the token's quad adds it: divided by 4 below
                if (kq == 0) pw[r * kF16Tok + kt] = p;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            // P.V: this lane's 4 tokens x 8 channels for each query head
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                const float4 pp = *reinterpret_cast<const float4*>(pw + r * kF16Tok + 4 * vg);
                const float pt[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t w[4] = {cur.v[u].x, cur.v[u].y, cur.v[u].z, cur.v[u].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        o[r][2 * j] = fmaf(pt[u], h2f(w[j] & 0xffffu), o[r][2 * j]);
                        o[r][2 * j + 1] = fmaf(pt[u], h2f(w[j] >> 16), o[r][2 * j + 1]);
                    }
                }
            }
            load_v(cur, nxt);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
            float x = o[r][c] + xor16_f(o[r][c]);
            x += __shfl_xor(x, 32, 64);
            o[r][c] = x;
        }
        const float l = wave_sum(lsum[r]) * 0.25f;
        if (lane < 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) sh_o[r][wave][8 * vc + c] = o[r][c];
        }
        if (lane == 0) {
            sh_m[r][wave] = m[r];
            sh_l[r][wave] = l;
            sh_m[r][kWaves + wave] = -INFINITY;   // no separate residual here
            sh_l[r][kWaves + wave] = 0.0f;
        }
    }
    __syncthreads();
    finish_block<NQ>(a, a.splits, split, qrow0, tag, sh_o, sh_m, sh_l);
}

hipError_t launch_decode_attn_fp16(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const dim3 grid((unsigned)a.splits, (unsigned)a.block_rows);
    switch (a.nq) {
        case 1: hipExtLaunchKernelGGL(attn_fp16_kernel<1>, grid, dim3(kBlock), 0, s, t0, t1, 0, a); break;
        case 2: hipExtLaunchKernelGGL(attn_fp16_kernel<2>, grid, dim3(kBlock), 0, s, t0, t1, 0, a); break;
        case 3: hipExtLaunchKernelGGL(attn_fp16_kernel<3>, grid, dim3(kBlock), 0, s, t0, t1, 0, a); break;
        case 4: hipExtLaunchKernelGGL(attn_fp16_kernel<4>, grid, dim3(kBlock), 0, s, t0, t1, 0, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kivi
