// kivi_attn.hip -- fused decode attention over the 2-bit cache (gfx950).
//
// One query per head attends over the dequantized history followed by the fp16
// residual: out = softmax(sm_scale * q.K^T) . V (error judged at the attention output:
// article "Your KV cache doesn't have a bit problem...", paragraph 3).  Keys are folded
// per token group: q.(z + c*s) = q.z + (q*s).c, computed once per group and channel;
// values per token: p*(z + c*s) = p*z + (p*s)*c.
//
// Work split: grid (splits, B*Hq).  A 256-thread workgroup owns one query row and a
// contiguous range of key groups; each of its 4 waves walks a quarter of that range
// with its own online softmax (log2 domain), the waves merge in LDS and the workgroup
// writes one partial (o[128], m, l).  The last workgroup of a row to finish (per-row
// arrival counter) merges the row's partials (log-sum-exp merge) and writes the output,
// so one launch does the whole call.  The split holding the last groups also reads the
// residual.
//
// Lane map inside a wave, per 32-token group: lane = 4*tp + qq handles tokens 2tp and
// 2tp+1 of the group and channels [32qq, 32qq+32); 8-byte code loads per token.
#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

constexpr int kWaves = kBlock / 64;
constexpr int kPart = kD + 2;   // floats per partial: o[128], m, l

__device__ __forceinline__ float code_f(uint32_t w, int c) {
    return (float)((w >> (2 * c)) & 3u);
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

__global__ __launch_bounds__(kBlock) void attn_split_kernel(AttnArgs a) {
    __shared__ float sh_o[kWaves][kD];
    __shared__ float sh_m[kWaves], sh_l[kWaves];

    const int split = blockIdx.x;
    const int64_t qrow = blockIdx.y;
    const int64_t b = qrow / a.q_heads;
    const int hq = (int)(qrow % a.q_heads);
    const int64_t kvrow = b * a.kv_heads + hq / a.ratio;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tp = lane >> 2, qq = lane & 3;

    float qv[32];
    load_q32(a.q + qrow * kD + qq * 32, a.sm_log2, qv);
    float o[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = 0.0f;
    float zacc = 0.0f, lsum = 0.0f, m = -INFINITY;

    const int n_groups = a.n_quant / kG;
    const int g_lo = split * a.groups_per_split;
    const int g_hi = min(n_groups, g_lo + a.groups_per_split);
    const int cnt = max(0, g_hi - g_lo);
    const int per_wave = (cnt + kWaves - 1) / kWaves;
    const int gb = g_lo + min(cnt, wave * per_wave);
    const int ge = g_lo + min(cnt, (wave + 1) * per_wave);

    const int64_t tok_base = kvrow * (int64_t)a.token_cap;
    const uint8_t* kc_row = a.k_codes + tok_base * kRowBytes;
    const uint8_t* vc_row = a.v_codes + tok_base * kRowBytes;
    const uint32_t* kp_row = reinterpret_cast<const uint32_t*>(a.k_sz) + kvrow * (int64_t)(a.token_cap / kG) * kD;
    const uint32_t* vp_row = reinterpret_cast<const uint32_t*>(a.v_sz) + tok_base * (kD / kG);

    for (int g = gb; g < ge; ++g) {
        const int64_t t0 = (int64_t)g * kG + 2 * tp;
        const uint2 kw0 = *reinterpret_cast<const uint2*>(kc_row + t0 * kRowBytes + qq * 8);
        const uint2 kw1 = *reinterpret_cast<const uint2*>(kc_row + (t0 + 1) * kRowBytes + qq * 8);
        const uint2 vw0 = *reinterpret_cast<const uint2*>(vc_row + t0 * kRowBytes + qq * 8);
        const uint2 vw1 = *reinterpret_cast<const uint2*>(vc_row + (t0 + 1) * kRowBytes + qq * 8);
        const uint32_t vp0 = vp_row[t0 * 4 + qq], vp1 = vp_row[(t0 + 1) * 4 + qq];
        const uint4* kp4 = reinterpret_cast<const uint4*>(kp_row + (int64_t)g * kD + qq * 32);
        float d0 = 0.0f, d1 = 0.0f, az = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 pr = kp4[i];
            const uint32_t pw[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int c = 4 * i + k;
                const float qs = qv[c] * h2f(pw[k] & 0xffffu);
                az = fmaf(qv[c], h2f(pw[k] >> 16), az);
                const uint32_t w0 = c < 16 ? kw0.x : kw0.y;
                const uint32_t w1 = c < 16 ? kw1.x : kw1.y;
                d0 = fmaf(qs, code_f(w0, c & 15), d0);
                d1 = fmaf(qs, code_f(w1, c & 15), d1);
            }
        }
        d0 = wave_sum_xor(d0, 1, 2);
        d1 = wave_sum_xor(d1, 1, 2);
        az = wave_sum_xor(az, 1, 2);
        const float l0 = az + d0, l1 = az + d1;
        const float m_new = fmaxf(m, wave_max_xor(fmaxf(l0, l1), 4, 32));
        const float alpha = (m == -INFINITY) ? 0.0f : exp2f(m - m_new);
        const float p0 = exp2f(l0 - m_new), p1 = exp2f(l1 - m_new);
        lsum = lsum * alpha + p0 + p1;
        const float w0 = p0 * h2f(vp0 & 0xffffu), w1 = p1 * h2f(vp1 & 0xffffu);
        zacc = zacc * alpha + p0 * h2f(vp0 >> 16) + p1 * h2f(vp1 >> 16);
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const uint32_t a0 = c < 16 ? vw0.x : vw0.y;
            const uint32_t a1 = c < 16 ? vw1.x : vw1.y;
            o[c] = fmaf(w1, code_f(a1, c & 15), fmaf(w0, code_f(a0, c & 15), o[c] * alpha));
        }
        m = m_new;
    }

    // fp16 residual, logical tokens [32*wave, 32*wave+32) of the ring, last split only
    if (split == a.splits - 1) {
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
            lsum = lsum * alpha + p0 + p1;
            zacc *= alpha;
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

    // wave result: sum over the 16 token-pair lanes of each channel quarter
    lsum = wave_sum_xor(lsum, 4, 32);
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] = wave_sum_xor(o[c] + zacc, 4, 32);
    if (tp == 0) {
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
        part[j] = O;
        if (j == 0) {
            part[kD] = M;
            part[kD + 1] = L;
        }
    }
    // The last workgroup of this row to finish merges every split's partial
    // (log-sum-exp merge) and writes the output; it then re-arms the row counter.
    __threadfence();
    __syncthreads();
    __shared__ bool sh_last;
    if (threadIdx.x == 0) sh_last = atomicAdd(&a.counters[qrow], 1u) == (unsigned)(a.splits - 1);
    __syncthreads();
    if (!sh_last) return;
    __threadfence();
    if (threadIdx.x < kD) {
        const int j = threadIdx.x;
        const float* rowp = a.ws + qrow * kPart;
        const int64_t stride = a.q_rows * kPart;
        float M = -INFINITY;
        for (int s = 0; s < a.splits; ++s) M = fmaxf(M, rowp[s * stride + kD]);
        float L = 0.0f, O = 0.0f;
        for (int s = 0; s < a.splits; ++s) {
            const float ms = rowp[s * stride + kD];
            if (ms == -INFINITY) continue;
            const float sc = exp2f(ms - M);
            L = fmaf(rowp[s * stride + kD + 1], sc, L);
            O = fmaf(rowp[s * stride + j], sc, O);
        }
        a.out[qrow * kD + j] = (uint16_t)f2h(O / L);
        if (j == 0) {
            if (a.lse != nullptr) a.lse[qrow] = (M + log2f(L)) * 0.69314718055994531f;
            a.counters[qrow] = 0u;
        }
    }
}

hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(attn_split_kernel, dim3((unsigned)a.splits, (unsigned)a.q_rows), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace kivi
