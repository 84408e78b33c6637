// kivi_attn_common.h -- pieces shared by the decode-attention kernels (gfx950).
//
// Every kernel keeps, per workgroup and query row, 2 * (its waves) softmax states in the log2
// domain (m, l, o[128] with o relative to 2^m): one per wave for the quantized history and
// one per wave for the fp16 residual.  finish_block() merges them (log-sum-exp), then either writes
// the output (one split) or a split partial; the last workgroup of a row to arrive merges
// the partials and writes the output, so one launch does the whole call.
#pragma once

#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

constexpr int kWaves = kBlock / 64;  // waves of a 256-thread workgroup (the fp16 comparator's)
constexpr int kSlots = 2 * kWaves;   // its softmax states per workgroup and row: quantized, residual
constexpr int kSqBlock = 64 * kSqWaves;   // threads of a single-query 2-bit attention workgroup
constexpr int kSqSlots = 2 * kSqWaves;
constexpr int kPart = kD + 2;        // floats per split partial: o[128], m, l

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// value of lane 4*(lane/4) + i, for CTRL = quad_perm [i, i, i, i]
template <int CTRL>
__device__ __forceinline__ float quad_bcast(float v) { return dpp_f<CTRL>(v); }

// (x & m) | o, one v_and_or_b32 when m and o sit in VGPRs (see in_vgpr).  Written in C, not
// inline asm, so that the compiler sees the instruction: its results feed matrix
// instructions, and the compiler must insert the wait states between a matrix instruction
// reading a register and a vector write to it.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) { return (x & m) | o; }
// A constant the compiler may not fold into literals: an empty asm statement (no instruction)
// pins it to a VGPR, so (x & m) | o selects one three-operand v_and_or_b32 instead of a
// v_and_b32 and a v_or_b32 with literal operands.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t c) {
    asm volatile("" : "+v"(c));
    return c;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// per-half unsigned maximum of two packed 16-bit pairs (one v_pk_max_u16)
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// sum over all 64 lanes (every lane gets it)
__device__ __forceinline__ float wave_sum(float v) {
    v = half_sum(v);
    return readlane_f(v, 0) + readlane_f(v, 32);
}
// sum / max over the 16 lanes of each DPP row (every lane gets its row's result)
__device__ __forceinline__ float row_sum(float v) {
    v += xor1_f(v);
    v += xor2_f(v);
    v += hmirror_f(v);
    return v + mirror_f(v);
}
__device__ __forceinline__ float row_max(float v) {
    v = __builtin_fmaxf(v, xor1_f(v));
    v = __builtin_fmaxf(v, xor2_f(v));
    v = __builtin_fmaxf(v, hmirror_f(v));
    return __builtin_fmaxf(v, mirror_f(v));
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
__device__ __forceinline__ void store_coherent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_coherent(uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A split partial's value with the call's tag: one 8-byte store, so a reader sees both or
// neither.
__device__ __forceinline__ uint64_t tagged(float v, uint32_t tag) {
    return (uint64_t)__builtin_bit_cast(uint32_t, v) | ((uint64_t)tag << 32);
}
// The tag of this call's split partials for counter row `counter`: one more than the epoch
// that the previous call's merging workgroup stored (0 in a cleared workspace).  Loaded when
// the workgroup starts; it is needed only when the workgroup ends.
__device__ __forceinline__ uint32_t partial_tag(const AttnArgs& a, int64_t counter) {
    return __hip_atomic_load(&a.counters[a.q_rows + counter], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
}
// The tag as a wave-uniform scalar, read where the caller places this call: after its first
// loads are issued, so that the wait for the tag's load overlaps the wait for them (a later
// first use, after the loop, could wait for every load in flight).
__device__ __forceinline__ uint32_t settle_tag(uint32_t v) {
    asm volatile("" : "+v"(v));
    return __builtin_amdgcn_readfirstlane(v);
}
// Polls of a partial value whose store has not landed yet (each after a short sleep).  The
// value was stored before its workgroup's arrival was counted, so it lands within a memory
// round trip; the bound only guarantees that the loop ends.
constexpr int kMaxPolls = 1 << 22;

// The (scale, zero) pairs of one value token, kD / GS of them, loaded at their own width (a
// wider load would read past the last token of the last row) and returned as one word per
// 32-channel block: word k is the pair of the group that holds channels 32k..32k+31.
template <int GS>
__device__ __forceinline__ uint4 load_value_pairs(const uint32_t* p) {
    if constexpr (GS == 32) {
        return *reinterpret_cast<const uint4*>(p);
    } else if constexpr (GS == 64) {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        return make_uint4(x.x, x.x, x.y, x.y);
    } else {
        const uint32_t x = *p;
        return make_uint4(x, x, x, x);
    }
}

// Grid of a decode-attention launch.  Workgroups go to the XCDs round-robin by linear id.
// Normally x = split: a row's splits spread over the XCDs.  In a ragged batch the
// sequences use different numbers of splits, so x = row instead (a sequence's kv heads are
// consecutive rows, so every XCD gets a share of every sequence whatever its length).
// The layout is chosen in launch code and kernels alike from a.seq_state.
inline dim3 attn_grid(const AttnArgs& a, int64_t rows) {
    return a.seq_state != nullptr ? dim3((unsigned)rows, (unsigned)a.splits) : dim3((unsigned)a.splits, (unsigned)rows);
}
__device__ __forceinline__ int grid_split(const AttnArgs& a) {
    return a.seq_state != nullptr ? (int)blockIdx.y : (int)blockIdx.x;
}
__device__ __forceinline__ int64_t grid_row(const AttnArgs& a) {
    return a.seq_state != nullptr ? (int64_t)blockIdx.x : (int64_t)blockIdx.y;
}

// The cache state one workgroup attends over: the call's, or (ragged batch) its sequence's,
// with the number of splits its row uses, its key groups per split and the split that also
// reads the residual.  A sequence state out of range gives an empty context (nothing is
// read) and sets the sequence's kSeqBadState flag.
//
// Ragged batch plan, the same in every workgroup: the batch's work W (key groups, with the
// residual counted as groups by its bytes) is read from all sequence states; a workgroup
// should take about W * rows_per_sequence / slot_budget of it, so that the whole batch fits
// one round of resident workgroups with even shares; a sequence uses floor(its work / that
// share) splits (at least one, at most the grid's).  Workgroups past their row's count do
// nothing.
struct RowState {
    int32_t n_quant, n_res, res_head, groups_per_split, res_split, splits;
};
// key groups the residual counts as (512 bytes per fp16 token against 96 per 2-bit token)
__device__ __forceinline__ int32_t residual_units(int32_t n_res) { return (n_res * 512 + 96 * kG - 1) / (96 * kG); }
// The batch's total work, by each wave: lane i reads sequence i's state (one coalesced
// 16-byte load per lane and 64 sequences), then a wave sum.
__device__ __forceinline__ int32_t batch_units(const AttnArgs& a, int64_t batch) {
    const int lane = threadIdx.x & 63;
    int32_t u = 0;
    for (int64_t b = lane; b < batch; b += 64) {
        const int4 st = *reinterpret_cast<const int4*>(a.seq_state + 4 * b);
        if (state_in_range(st.x, st.y, st.z, a.token_cap, a.residual_cap, a.group)) u += st.x / kG + residual_units(st.y);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) u += __shfl_xor(u, m, 64);
    return __builtin_amdgcn_readfirstlane(u);
}
__device__ __forceinline__ RowState row_state(const AttnArgs& a, int64_t kvrow, int split) {
    if (a.seq_state == nullptr) return {a.n_quant, a.n_res, a.res_head, a.groups_per_split, a.splits - 1, a.splits};
    int32_t* s = a.seq_state + 4 * (kvrow / a.kv_heads);
    int32_t nq = s[0], nr = s[1], rh = s[2];
    if (!state_in_range(nq, nr, rh, a.token_cap, a.residual_cap, a.group)) {
        if (split == 0 && threadIdx.x == 0)
            __hip_atomic_fetch_or(&s[3], kSeqBadState, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        nq = nr = rh = 0;
    }
    const int32_t units = nq / kG + residual_units(nr);
    const int64_t batch = a.q_rows / a.q_heads;
    const int64_t total = batch_units(a, batch);
    const int64_t rows_per_seq = a.block_rows / batch;
    const int64_t share = max((int64_t)1, (total * rows_per_seq + a.slot_budget - 1) / a.slot_budget);
    const int32_t active = (int32_t)max((int64_t)1, min((int64_t)a.splits, (int64_t)units / share));
    return {nq, nr, rh, (units + active - 1) / active, active - 1, active};
}

// Softmax states of query rows qrow0..qrow0+NQ-1 over the fp16 residual ring.  Called by one
// whole wave of a WAVES-wave workgroup; wave w takes the ring's logical tokens
// [32w + 32*WAVES*i, 32w + 32*WAVES*i + 32).  Per such
// chunk, two phases:
//  * logits: lane 4*tp + qq holds tokens 2tp, 2tp+1 and channels [32qq, 32qq+32) and forms
//    q.k with v_dot2_f32_f16 on packed halves for every row; the chunk's probabilities go to
//    LDS (o_dst, channels 0..31 of each row, as scratch);
//  * P.V, channel-parallel: lane l accumulates channels 2l, 2l+1 of every row over the
//    chunk's tokens (token rows loaded 256 bytes per instruction, probabilities read from LDS
//    as broadcasts), so no cross-lane sums are needed.
// Row r's o (relative to 2^m[r]) ends in o_dst[r*o_stride + c]; m[r] = -inf and l[r] = 0 when
// the wave has no residual token.  In a fused decode step the last residual token is the new
// one, read from k_new / v_new.
template <int NQ, int WAVES = kWaves>
__device__ void residual_states(const AttnArgs& a, const RowState& rs, int64_t qrow0, int64_t kvrow, int wave,
                                float* o_dst, int o_stride, float (&mr)[NQ], float (&lr)[NQ]) {
    const int lane = threadIdx.x & 63, tp = lane >> 2, qq = lane & 3;
    float o[NQ][2];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        mr[r] = -INFINITY;
        lr[r] = 0.0f;
        o[r][0] = o[r][1] = 0.0f;
    }
    auto token_slot = [&](int i) { return (rs.res_head + i) % a.residual_cap; };
    auto is_new = [&](int i) { return a.k_new != nullptr && i == rs.n_res - 1; };
    for (int base = wave * kG; base < rs.n_res; base += WAVES * kG) {
        // ---- logits of tokens 2tp, 2tp+1 for every row
        const int i0 = base + 2 * tp, i1 = i0 + 1;
        const bool ok0 = i0 < rs.n_res, ok1 = i1 < rs.n_res;
        const int j0 = ok0 ? i0 : 0, j1 = ok1 ? i1 : 0;
        const int64_t rn = kvrow * kD + qq * 32;
        const uint4* k0 = reinterpret_cast<const uint4*>(
            is_new(j0) ? a.k_new + rn : a.k_res + (kvrow * a.residual_cap + token_slot(j0)) * kD + qq * 32);
        const uint4* k1 = reinterpret_cast<const uint4*>(
            is_new(j1) ? a.k_new + rn : a.k_res + (kvrow * a.residual_cap + token_slot(j1)) * kD + qq * 32);
        uint4 kx0[4], kx1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kx0[i] = k0[i];
            kx1[i] = k1[i];
        }
        float al[NQ];
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            // q.k on packed halves: each fp16 product is exact in fp32, summed in fp32
            const uint4* qp = reinterpret_cast<const uint4*>(a.q + (qrow0 + r) * kD + qq * 32);
            float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 qx = qp[i];
                const uint32_t qh[4] = {qx.x, qx.y, qx.z, qx.w};
                const uint32_t w0[4] = {kx0[i].x, kx0[i].y, kx0[i].z, kx0[i].w};
                const uint32_t w1[4] = {kx1[i].x, kx1[i].y, kx1[i].z, kx1[i].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    d0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qh[k]), __builtin_bit_cast(h2v, w0[k]), d0, false);
                    d1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, qh[k]), __builtin_bit_cast(h2v, w1[k]), d1, false);
                }
            }
            d0 = quad_sum(d0) * a.sm_log2;   // over the 4 channel quarters
            d1 = quad_sum(d1) * a.sm_log2;
            const float l0 = ok0 ? d0 : -INFINITY, l1 = ok1 ? d1 : -INFINITY;
            const float m_new = fmaxf(mr[r], wave_max_quads(fmaxf(l0, l1)));
            al[r] = (mr[r] == -INFINITY) ? 0.0f : exp2f(mr[r] - m_new);
            const float p0 = ok0 ? exp2f(l0 - m_new) : 0.0f;
            const float p1 = ok1 ? exp2f(l1 - m_new) : 0.0f;
            lr[r] = lr[r] * al[r] + wave_sum(qq == 0 ? p0 + p1 : 0.0f);   // one share per token pair
            mr[r] = m_new;
            if (qq == 0) {
                o_dst[r * o_stride + 2 * tp] = p0;
                o_dst[r * o_stride + 2 * tp + 1] = p1;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- P.V: lane l takes channels 2l, 2l+1 of the chunk's 32 token rows
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            o[r][0] *= al[r];
            o[r][1] *= al[r];
        }
        const int nt = min(kG, rs.n_res - base);
        for (int t0 = 0; t0 < nt; t0 += 8) {
            uint32_t vv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = base + min(t0 + u, nt - 1);
                const uint16_t* row = is_new(i) ? a.v_new + kvrow * kD : a.v_res + (kvrow * a.residual_cap + token_slot(i)) * kD;
                vv[u] = reinterpret_cast<const uint32_t*>(row)[lane];
            }
#pragma unroll
            for (int r = 0; r < NQ; ++r) {
                const float4 pa = *reinterpret_cast<const float4*>(o_dst + r * o_stride + t0);
                const float4 pb = *reinterpret_cast<const float4*>(o_dst + r * o_stride + t0 + 4);
                const float pt[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float pu = t0 + u < nt ? pt[u] : 0.0f;
                    o[r][0] = fmaf(pu, h2f(vv[u] & 0xffffu), o[r][0]);
                    o[r][1] = fmaf(pu, h2f(vv[u] >> 16), o[r][1]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (wave * kG < rs.n_res) {
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            o_dst[r * o_stride + 2 * lane] = o[r][0];
            o_dst[r * o_stride + 2 * lane + 1] = o[r][1];
        }
    }
}

// Fused decode step: threads 0..31 of the calling workgroup store the new token (k_new /
// v_new of KV row kvrow) into its ring slot.  Exactly one workgroup per KV row calls it;
// no workgroup of the launch reads that slot (attention takes the token from k_new / v_new).
__device__ __forceinline__ void store_new_token(const AttnArgs& a, int64_t kvrow) {
    if (threadIdx.x < 32) {
        const int c = threadIdx.x & 15;
        const uint16_t* src = (threadIdx.x < 16 ? a.k_new : a.v_new) + kvrow * kD;
        uint16_t* dst = (threadIdx.x < 16 ? a.k_ring : a.v_ring) + (kvrow * a.residual_cap + a.new_slot) * kD;
        reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
    }
}

// Log-sum-exp merge of the split partials of query rows qrow0..qrow0+NQ-1, by the whole
// workgroup, with each thread's coherent loads issued together: a thread merges, for one
// (row, channel), every lpp-th split online (lpp = THREADS / 128 for one row, else 1), and
// the lpp threads of a channel combine in LDS.  out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// lse = (M + log2 L) ln 2.  Re-arms the arrival counter.
constexpr int kMergeBatch = 8;
template <int NQ, int THREADS = kBlock>
__device__ __forceinline__ void merge_rows(const AttnArgs& a, int splits, int64_t qrow0, int64_t counter,
                                           uint32_t tag) {
    constexpr int kLpp = NQ == 1 ? THREADS / kD : 1;
    static_assert(NQ != 1 || (THREADS % kD == 0 && kLpp >= 2), "one row needs whole multiples of 128 threads");
    __shared__ float sh_mo[kLpp > 1 ? kLpp - 1 : 1][kD + 2];
    const int t = threadIdx.x, sub = kLpp > 1 ? t / kD : 0;
    const int64_t stride = a.q_rows * kPart;
    for (int idx = kLpp > 1 ? (t % kD) : t; idx < NQ * kD; idx += THREADS / kLpp) {
        const int r = idx / kD, j = idx % kD;
        uint64_t* rowp = a.ws + (qrow0 + r) * kPart;
        // a value of this call: loaded again until its tag is this call's
        auto settle = [&](uint64_t* p, uint64_t v) {
            for (int n = 0; (uint32_t)(v >> 32) != tag && n < kMaxPolls; ++n) {
                __builtin_amdgcn_s_sleep(1);
                v = load_coherent(p);
            }
            return __builtin_bit_cast(float, (uint32_t)v);
        };
        float M = -INFINITY, L = 0.0f, O = 0.0f;
        for (int s0 = sub; s0 < splits; s0 += kLpp * kMergeBatch) {
            uint64_t mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch];
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {   // every load first, then the checks
                const int s = s0 + kLpp * u;
                if (s < splits) {
                    uint64_t* ps = rowp + s * stride;
                    mv[u] = load_coherent(ps + kD);
                    lv[u] = load_coherent(ps + kD + 1);
                    ov[u] = load_coherent(ps + j);
                }
            }
            float ms[kMergeBatch], ls[kMergeBatch], os[kMergeBatch];
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const int s = s0 + kLpp * u;
                ms[u] = -INFINITY;
                ls[u] = os[u] = 0.0f;
                if (s < splits) {
                    uint64_t* ps = rowp + s * stride;
                    ms[u] = settle(ps + kD, mv[u]);
                    ls[u] = settle(ps + kD + 1, lv[u]);
                    os[u] = settle(ps + j, ov[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                if (ms[u] == -INFINITY) continue;
                const float mn = fmaxf(M, ms[u]);
                const float al = exp2f(M - mn), be = exp2f(ms[u] - mn);   // M = -inf gives al = 0
                L = fmaf(L, al, ls[u] * be);
                O = fmaf(O, al, os[u] * be);
                M = mn;
            }
        }
        if (kLpp > 1) {   // one iteration per thread here: the barrier is reached by all
            if (sub > 0) {
                sh_mo[sub - 1][j] = O;
                if (j == 0) {
                    sh_mo[sub - 1][kD] = M;
                    sh_mo[sub - 1][kD + 1] = L;
                }
            }
            __syncthreads();
            if (sub > 0) return;
#pragma unroll
            for (int k = 0; k < kLpp - 1; ++k) {
                const float m1 = sh_mo[k][kD], l1 = sh_mo[k][kD + 1], o1 = sh_mo[k][j];
                const float mn = fmaxf(M, m1);
                const float al = M == -INFINITY ? 0.0f : exp2f(M - mn), be = m1 == -INFINITY ? 0.0f : exp2f(m1 - mn);
                L = fmaf(L, al, l1 * be);
                O = fmaf(O, al, o1 * be);
                M = mn;
            }
        }
        a.out[(qrow0 + r) * kD + j] = (uint16_t)f2h(L > 0.0f ? O / L : 0.0f);
        if (j == 0 && a.lse != nullptr) a.lse[qrow0 + r] = (M + log2f(L)) * 0.69314718055994531f;
    }
    if (t == 0) {
        a.counters[counter] = 0u;
        a.counters[a.q_rows + counter] = tag;   // the next call's partials carry tag + 1
    }
}

// End of a WAVES-wave workgroup: merge its 2*WAVES states per row (empty states skipped), then write the
// output directly (one split) or the split partial, and let the last workgroup of the row
// group to arrive merge the partials.  Every partial value carries the call's tag (tag, from
// partial_tag at the workgroup's start), so the merging workgroup, which loads after its own
// arrival returned the final count, tells a value of this call from a stale one.
template <int NQ, int WAVES = kWaves>
__device__ __forceinline__ void finish_block(const AttnArgs& a, int splits, int split, int64_t qrow0, int64_t counter,
                                             uint32_t tag, const float (*sh_o)[2 * WAVES][kD],
                                             const float (*sh_m)[2 * WAVES], const float (*sh_l)[2 * WAVES]) {
    constexpr int kS = 2 * WAVES;
    // The arrival is counted first, by the last wave, before the merge below and the partial
    // stores: its round trip overlaps them, and the merging workgroup checks each value's tag
    // and loads a value again until its store has landed.  A wave's memory operations
    // complete in issue order, so the arrival is counted by the wave with the least other
    // work here (none in a 12-wave workgroup with one query row).
    constexpr int kArrive = 64 * (WAVES - 1);
    uint32_t arrived = 0;
    if (splits > 1 && threadIdx.x == kArrive)
        arrived = __hip_atomic_fetch_add(&a.counters[counter], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int idx = threadIdx.x; idx < NQ * kD; idx += 64 * WAVES) {
        const int r = idx / kD, j = idx % kD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kS; ++w) M = fmaxf(M, sh_m[r][w]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kS; ++w) {
            if (sh_m[r][w] == -INFINITY) continue;
            const float sc = exp2f(sh_m[r][w] - M);
            L = fmaf(sh_l[r][w], sc, L);
            O = fmaf(sh_o[r][w][j], sc, O);
        }
        if (splits == 1) {
            // an empty context (a ragged batch's empty sequence) gives out = 0, lse = -inf
            a.out[(qrow0 + r) * kD + j] = (uint16_t)f2h(L > 0.0f ? O / L : 0.0f);
            if (j == 0 && a.lse != nullptr) a.lse[qrow0 + r] = (M + log2f(L)) * 0.69314718055994531f;
        } else {
            uint64_t* part = a.ws + ((int64_t)split * a.q_rows + qrow0 + r) * kPart;
            store_coherent(&part[j], tagged(O, tag));
            if (j == 0) {
                store_coherent(&part[kD], tagged(M, tag));
                store_coherent(&part[kD + 1], tagged(L, tag));
            }
        }
    }
    if (splits == 1) return;
    __shared__ bool sh_last;
    if (threadIdx.x == kArrive) sh_last = arrived == (unsigned)(splits - 1);
    __syncthreads();
    if (sh_last) merge_rows<NQ, 64 * WAVES>(a, splits, qrow0, counter, tag);
}

}  // namespace kivi
