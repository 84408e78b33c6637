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
    v = fmax_ieee(v, perm_f<0xB1>(v));
    v = fmax_ieee(v, perm_f<0x4E>(v));
    v = fmax_ieee(v, perm_f<0x141>(v));
    return fmax_ieee(v, perm_f<0x140>(v));
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
// The tag of this call's split partials for query rows qrow0..qrow0+NQ-1: one more than the
// largest call epoch of those rows.  A row's epoch is the tag of the last partials merged for
// it (0 in a cleared workspace), whichever kernel wrote them, so the tag is above every tag
// left in the rows' partial slots, also when entry points that group query rows differently
// (one row per workgroup, or a KV head's query group) share a workspace.  The epochs are
// loaded when the workgroup starts; they are needed only when it ends (settle_tag).
template <int NQ>
struct TagLoads {
    uint32_t e[NQ];
};
template <int NQ>
__device__ __forceinline__ TagLoads<NQ> partial_tag(const AttnArgs& a, int64_t qrow0) {
    TagLoads<NQ> t;
#pragma unroll
    for (int r = 0; r < NQ; ++r)
        t.e[r] = __hip_atomic_load(&a.counters[a.q_rows + qrow0 + r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return t;
}
// The tag as a wave-uniform scalar, read where the caller places this call: after its first
// loads are issued, so that the wait for the epochs overlaps the wait for them (a later first
// use, after the loop, could wait for every load in flight).
template <int NQ>
__device__ __forceinline__ uint32_t settle_tag(TagLoads<NQ> t) {
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        uint32_t v = t.e[r];
        asm volatile("" : "+v"(v));
        m = max(m, v);
    }
    // (pinned to a scalar register here: otherwise the compiler may move the read down to the
    // tag's first use, after the loop, and hold the epochs in a vector register until then)
    uint32_t tag = __builtin_amdgcn_readfirstlane(m) + 1u;
    asm volatile("" : "+s"(tag));
    return tag;
}
// Polls of a partial value whose store has not landed yet (each after a short sleep).  The
// value was stored before its workgroup's arrival was counted, so it lands within a memory
// round trip; the bound only guarantees that the loop ends.  A merge that reaches it writes
// NaN for the row and sets kWsPollTimeout in the workspace's status word.
constexpr int kMaxPolls = 1 << 22;
constexpr uint32_t kWsPollTimeout = 1u;   // the status word's bit (KIVI_WS_POLL_TIMEOUT)

// The (scale, zero) pairs of one value token, kD / GS of them, loaded at their own width (a
// wider load would read past the last token of the last row) and returned as one word per
// 32-channel block: word k is the pair of the group that holds channels 32k..32k+31.
template <int GS, bool STREAM>
__device__ __forceinline__ uint4 load_value_pairs(const uint32_t* p) {
    if constexpr (GS == 32) {
        return STREAM ? stream_load16(p) : *reinterpret_cast<const uint4*>(p);
    } else if constexpr (GS == 64) {
        const uint2 x = STREAM ? stream_load8(p) : *reinterpret_cast<const uint2*>(p);
        return make_uint4(x.x, x.x, x.y, x.y);
    } else {
        const uint32_t x = STREAM ? stream_load4(p) : *p;
        return make_uint4(x, x, x, x);
    }
}

// Wave priority from the loop iterations a wave has left (s_setprio takes an immediate):
// waves with more left issue first, in four steps that close in towards the end.
__device__ __forceinline__ void set_priority_for(int left) {
    if (left >= 6) __builtin_amdgcn_s_setprio(3);
    else if (left >= 4) __builtin_amdgcn_s_setprio(2);
    else if (left >= 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// The cache state one workgroup attends over, with the number of splits its row uses, its
// key groups per split and the split that also reads the residual.
struct RowState {
    int32_t n_quant, n_res, res_head, groups_per_split, res_split, splits;
};
// One workgroup's work: its grid row (a query row, or a query-group row), its split of that
// row's context, and (ragged batch) the state of the row's sequence; split < 0: no work.
struct WorkItem {
    int64_t row;
    int split;
    RowState rs;
};

// Grid of a decode-attention launch.  Uniform batch: x = split, y = row (workgroups go to the
// XCDs round-robin by linear id, so a row's splits spread over them).  Ragged batch: one
// dimension, one workgroup per item of the plan below, at most max(slot_budget, rows) of them.
inline dim3 attn_grid(const AttnArgs& a, int64_t rows) {
    if (a.seq_state != nullptr) return dim3((unsigned)(rows > a.slot_budget ? rows : a.slot_budget));
    return dim3((unsigned)a.splits, (unsigned)rows);
}
__device__ __forceinline__ RowState row_state(const AttnArgs& a) {
    return {a.n_quant, a.n_res, a.res_head, a.groups_per_split, a.splits - 1, a.splits};
}

// key groups the residual counts as (512 bytes per fp16 token against 96 per 2-bit token)
__device__ __forceinline__ int32_t residual_units(int32_t n_res) { return (n_res * 512 + 96 * kG - 1) / (96 * kG); }
// work of sequence b in key groups (its residual counted by its bytes); 0 for a state out of range
__device__ __forceinline__ int32_t seq_units(const AttnArgs& a, int64_t b) {
    const int4 st = *reinterpret_cast<const int4*>(a.seq_state + 4 * b);
    return state_in_range(st.x, st.y, st.z, a.token_cap, a.residual_cap, a.group) ? st.x / kG + residual_units(st.y) : 0;
}
// Integer reductions and scan over the wave without LDS traffic (the plan below runs them
// back to back, so each step's latency counts): DPP inside 16-lane rows, then readlane of
// the four rows' results.
template <int CTRL>
__device__ __forceinline__ int32_t dpp_i(int32_t v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }
__device__ __forceinline__ int32_t wave_sum(int32_t v) {
    v += dpp_i<0xB1>(v);    // lane^1
    v += dpp_i<0x4E>(v);    // lane^2
    v += dpp_i<0x141>(v);   // the other quad of the half-row
    v += dpp_i<0x140>(v);   // the other half-row
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {
    v = max(v, dpp_i<0xB1>(v));
    v = max(v, dpp_i<0x4E>(v));
    v = max(v, dpp_i<0x141>(v));
    v = max(v, dpp_i<0x140>(v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// sum of values below 2^47 per lane, as two 32-bit sums of 16-bit and 31-bit parts
__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
    const int64_t lo = wave_sum((int32_t)(v & 0xffff)), hi = wave_sum((int32_t)(v >> 16));
    return (hi << 16) + lo;
}
// inclusive prefix sum over the 64 lanes: inside each 16-lane row (shifts right by 1, 2, 4
// and 8; lanes without a source add 0), then the totals of the rows below
__device__ __forceinline__ int32_t wave_prefix(int32_t v) {
    v += dpp_i<0x111>(v);
    v += dpp_i<0x112>(v);
    v += dpp_i<0x114>(v);
    v += dpp_i<0x118>(v);
    const int32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
                  r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
// ceil(u / s), u < 2^24: the product with the reciprocal is within one of the quotient
__device__ __forceinline__ int32_t ceil_div_small(int32_t u, int32_t s, float rcp) {
    int32_t q = (int32_t)((float)u * rcp);
    q += (int32_t)(q * s < u);
    q -= (int32_t)((q > 0) & ((q - 1) * s >= u));   // (bitwise: no branches)
    return q;
}
// splits of a sequence of u units at a share of s units: ceil(u / s), at least 1, at most cap
__device__ __forceinline__ int32_t seq_splits(int32_t u, int32_t s, float rcp, int32_t cap) {
    return min(cap, max(1, ceil_div_small(u, s, rcp)));
}

// Ragged batch plan, computed alike by every wave of every workgroup from the sequence states
// (device memory, so a serving loop steps them without the host).  Sequence b's work u_b is
// its key groups plus its residual counted as groups by its bytes.  For a share s, sequence b
// takes a_b = ceil(u_b / s) splits (at least one, at most the workspace's a.splits) on each of
// its rows_per_seq grid rows; the plan uses the smallest s for which the items, rows_per_seq *
// sum a_b, fit the resident workgroups (a.slot_budget), found by bisection between
// rows_per_seq*W/budget (below it the items cannot fit) and rows_per_seq*W/(budget -
// rows_per_seq*batch) (every sequence rounds up by less than one split).  So the whole batch
// runs in one round and no item exceeds the share.
//
// Placement.  The hardware deals a launch's workgroups to the XCDs in turn and, inside an
// XCD, to its CUs in turn, so workgroups i, i + kCus, i + 2 kCus, ... share a CU.  With up
// to 64 sequences the items are ranked by size (the sequence's groups per split, largest
// first; a sequence's items are consecutive ranks, split-major, its rows one after another)
// and dealt in a snake: rounds of kCus workgroups take ranks in order, every other round in
// reverse, so each CU gets a large, a middle and a small item instead of whatever sizes
// sequence order puts together.  Larger batches take the items in sequence order.  Either
// way workgroup i finds its item with a prefix sum over the wave, and workgroups past the
// last item have none.  A state out of range counts as empty (one split that reads nothing)
// and its split-0 first-row item sets the sequence's kSeqBadState flag.
constexpr int kPlanRegs = 4;    // sequences lane + 64j, j < kPlanRegs, keep their work in registers
// One wave's plan (lds: 128 free words)
__device__ __forceinline__ WorkItem ragged_plan(const AttnArgs& a, int32_t* lds) {
    const int lane = threadIdx.x & 63;
    // (the host keeps a ragged grid's rows below 2^31: 32-bit divisions)
    const int32_t batch = (int32_t)((uint32_t)a.q_rows / (uint32_t)a.q_heads);
    const int32_t rps = (int32_t)((uint32_t)a.block_rows / (uint32_t)batch);
    const int32_t cap = a.splits;
    // the share of the last ragged call on this workspace: a starting point (checked below)
    const int32_t hint = (int32_t)a.status[1];
    // the lane's own sequence's state stays in registers for the item's state below
    int4 st0 = make_int4(0, 0, 0, 0);
    if (lane < batch) st0 = *reinterpret_cast<const int4*>(a.seq_state + 4 * lane);
    const bool ok0 = lane < batch && state_in_range(st0.x, st0.y, st0.z, a.token_cap, a.residual_cap, a.group);
    int32_t u[kPlanRegs];
    u[0] = ok0 ? st0.x / kG + residual_units(st0.y) : 0;
    int64_t w = u[0];
    int32_t umax = u[0];
#pragma unroll
    for (int j = 1; j < kPlanRegs; ++j) {
        const int64_t b = lane + 64 * j;
        u[j] = b < batch ? seq_units(a, b) : 0;
        w += u[j];
        umax = max(umax, u[j]);
    }
    for (int64_t b = lane + 64 * kPlanRegs; b < batch; b += 64) {
        const int32_t x = seq_units(a, b);
        w += x;
        umax = max(umax, x);
    }
    const int64_t total = wave_sum64(w) * rps;   // item-units of the whole batch
    umax = max(1, wave_max(umax));
    // most splits (summed over sequences) that fit the budget
    const int32_t most = a.slot_budget / rps;
    // sum of a_b at share s, saturated past `most` (only the comparison with it matters)
    auto splits_at = [&](int32_t s) {
        const float rcp = __builtin_amdgcn_rcpf((float)s);
        int32_t c = lane < batch ? seq_splits(u[0], s, rcp, cap) : 0;
        if (batch > 64) {
#pragma unroll
            for (int j = 1; j < kPlanRegs; ++j) {
                const int32_t x = seq_splits(u[j], s, rcp, cap);
                c += lane + 64 * j < batch ? x : 0;
            }
            for (int64_t b = lane + 64 * kPlanRegs; b < batch && c <= most; b += 64)
                c += seq_splits(seq_units(a, b), s, rcp, cap);
        }
        return wave_sum(min(c, most + 1));
    };
    int64_t hi = umax;
    const int64_t room = (int64_t)a.slot_budget - (int64_t)rps * batch;
    if (room > 0) hi = min(hi, max((int64_t)1, (total + room - 1) / room));
    int32_t lo = (int32_t)min(hi, max((int64_t)1, (total + a.slot_budget - 1) / a.slot_budget));
    // in a decode loop the smallest share that fits seldom moves: test the last call's first
    // (whatever the word holds, the bisection below still finds the smallest share that fits)
    if (hint >= lo && hint <= hi) {
        if (splits_at(hint) <= most) {
            hi = hint;
            if (hint > lo && splits_at(hint - 1) > most) lo = hint;
        } else {
            lo = hint + 1;
        }
    }
    while (lo < hi) {
        const int32_t mid = lo + (int32_t)(hi - lo) / 2;
        if (splits_at(mid) <= most) hi = mid;
        else lo = mid + 1;
    }
    const int32_t share = __builtin_amdgcn_readfirstlane(lo);
    const float rcp = __builtin_amdgcn_rcpf((float)share);
    if (blockIdx.x == 0 && lane == 0) a.status[1] = (uint32_t)share;   // the next call's starting point

    // the item's sequence k (a lane of chunk 0, or of a later chunk), its split and row
    // (items are fewer than 2^31: 32-bit divisions)
    auto item = [&](int64_t seq, int32_t a_k, int32_t u_k, int32_t local, int4 st) -> WorkItem {
        const int split = (int)((uint32_t)local / (uint32_t)rps);
        const int32_t r = local - split * rps;
        int32_t nq = st.x, nr = st.y, rh = st.z;
        if (!state_in_range(nq, nr, rh, a.token_cap, a.residual_cap, a.group)) {
            if (split == 0 && r == 0 && threadIdx.x == 0)
                __hip_atomic_fetch_or(&a.seq_state[4 * seq + 3], kSeqBadState, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            nq = nr = rh = 0;
        }
        return {seq * rps + r, split, {nq, nr, rh, (u_k + a_k - 1) / a_k, a_k - 1, a_k}};
    };
    auto lane_state = [&](int k) {
        return make_int4(__builtin_amdgcn_readlane(st0.x, k), __builtin_amdgcn_readlane(st0.y, k),
                         __builtin_amdgcn_readlane(st0.z, k), 0);
    };
    const int64_t g = blockIdx.x;
    if (batch <= 64) {
        // items ranked by size: sequence b's first rank is the items of every sequence with
        // larger items, or equal ones and a lower index
        const bool live = lane < batch;
        const int32_t ab = live ? seq_splits(u[0], share, rcp, cap) : 0;
        const int32_t key = live ? (u[0] + ab - 1) / ab : -1;
        const int32_t cnt = ab * rps;
        // (every lane reads every entry: broadcast LDS reads; a wave's LDS accesses complete in
        // issue order)
        lds[lane] = key;
        lds[64 + lane] = cnt;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // four entries per read, all reads unrolled so that they overlap (entries past the
        // batch hold key -1 and count 0 and add nothing)
        int32_t start = 0;
        const int4* lk = reinterpret_cast<const int4*>(lds);
        const int4* lc = reinterpret_cast<const int4*>(lds + 64);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int4 k4 = lk[q], c4 = lc[q];
            const int32_t kq[4] = {k4.x, k4.y, k4.z, k4.w}, cq[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // (bitwise, so that the compiler emits selects, not a branch per entry)
                const bool ahead = (kq[e] > key) | ((kq[e] == key) & (4 * q + e < lane));
                start += ahead ? cq[e] : 0;
            }
        }
        // this workgroup's rank: its position, reversed inside every odd whole round of kCus
        const int64_t round = g / kCus;
        const int64_t rank = (round & 1) && (round + 1) * kCus <= (int64_t)gridDim.x ? round * kCus + (kCus - 1) - (g - round * kCus) : g;
        const uint64_t hit = __ballot(live && start <= rank && rank < start + cnt);
        if (hit == 0) return {0, -1, {0, 0, 0, 0, 0, 0}};   // past the last item
        const int k = __builtin_ctzll(hit);
        const int32_t a_k = __builtin_amdgcn_readlane(ab, k), u_k = __builtin_amdgcn_readlane(u[0], k);
        return item(k, a_k, u_k, (int32_t)rank - __builtin_amdgcn_readlane(start, k), lane_state(k));
    }
    // more sequences: items in sequence order; global split index gs, row r of the sequence
    const int64_t gs = (uint32_t)g / (uint32_t)rps;
    const int32_t r = (int32_t)(g - gs * rps);
    int64_t before = 0;   // splits of the sequences before this 64-sequence chunk
    for (int64_t b0 = 0; b0 < batch; b0 += 64) {
        const int64_t b = b0 + lane;
        const int64_t j = b0 / 64;
        int32_t ub = 0;
#pragma unroll
        for (int t = 0; t < kPlanRegs; ++t)
            if (t == j) ub = u[t];
        if (j >= kPlanRegs && b < batch) ub = seq_units(a, b);
        const int32_t ab = b < batch ? seq_splits(ub, share, rcp, cap) : 0;
        const int32_t incl = wave_prefix(ab);  // inclusive prefix of a_b over the chunk
        // sequences of the chunk that end at or before split gs
        const uint64_t done = __ballot(b < batch && before + incl <= gs);
        const int k = __popcll(done);
        const int64_t last = min((int64_t)64, batch - b0);
        if (k < last) {
            // (wave-uniform; kept in scalar registers through the kernel)
            const int32_t a_k = __builtin_amdgcn_readlane(ab, k);
            const int32_t u_k = __builtin_amdgcn_readlane(ub, k);
            const int32_t incl_k = __builtin_amdgcn_readlane(incl, k);
            const int64_t seq = b0 + k;
            const int32_t local = (int32_t)(gs - (before + incl_k - a_k)) * rps + r;
            return item(seq, a_k, u_k, local, j == 0 ? lane_state(k) : *reinterpret_cast<const int4*>(a.seq_state + 4 * seq));
        }
        before += __builtin_amdgcn_readlane(incl, 63);
    }
    return {0, -1, {0, 0, 0, 0, 0, 0}};   // past the last item
}

// The workgroup's item: wave 0 plans (the plan is the same in every wave, and every wave's
// vector instructions share the CU's SIMDs with the other workgroups' waves) and leaves the
// item in LDS for the others.  lds: 128 words that nothing else uses until the plan is done;
// the second barrier keeps every wave's reads ahead of any later write to them.
__device__ __forceinline__ WorkItem ragged_item(const AttnArgs& a, int32_t* lds) {
    if (threadIdx.x < 64) {
        const WorkItem wi = ragged_plan(a, lds);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (threadIdx.x == 0) {
            lds[0] = (int32_t)(uint32_t)(uint64_t)wi.row;
            lds[1] = (int32_t)(uint32_t)((uint64_t)wi.row >> 32);
            lds[2] = wi.split;
            lds[3] = wi.rs.n_quant;
            lds[4] = wi.rs.n_res;
            lds[5] = wi.rs.res_head;
            lds[6] = wi.rs.groups_per_split;
            lds[7] = wi.rs.res_split;
            lds[8] = wi.rs.splits;
        }
    }
    __syncthreads();
    int32_t v[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) v[i] = __builtin_amdgcn_readfirstlane(lds[i]);
    __syncthreads();
    return {(int64_t)(((uint64_t)(uint32_t)v[1] << 32) | (uint32_t)v[0]), v[2], {v[3], v[4], v[5], v[6], v[7], v[8]}};
}

// The work of this workgroup: uniform batch, row y and split x of the grid (the state is the
// call's, row_state); ragged batch, the plan's item (lds: as ragged_item's).
template <bool RAGGED>
__device__ __forceinline__ WorkItem work_item(const AttnArgs& a, int32_t* lds) {
    if constexpr (RAGGED) return ragged_item(a, lds);
    else return {(int64_t)blockIdx.y, (int)blockIdx.x, {0, 0, 0, 0, 0, 0}};
}

// Softmax states of query rows qrow0..qrow0+NQ-1 over the fp16 residual ring.  Called by one
// whole wave of a WAVES-wave workgroup; wave w takes the ring's logical tokens
// [32w + 32*WAVES*i, 32w + 32*WAVES*i + 32).  Per such
// chunk, two phases:
//  * logits: q.K^T on the matrix cores, 16 tokens per instruction (rows: the queries), the
//    softmax over the lanes that hold the chunk's tokens; the chunk's weights go to LDS as
//    fp16 (o_dst, the first 64 bytes of each row, as scratch);
//  * P.V, channel-parallel: lane l accumulates channels 2l, 2l+1 of every row over the
//    chunk's tokens (token rows loaded 256 bytes per instruction, probabilities read from LDS
//    as broadcasts), so no cross-lane sums are needed.
// Row r's o (relative to 2^m[r]) ends in o_dst[r*o_stride + c]; m[r] = -inf and l[r] = 0 when
// the wave has no residual token.  In a fused decode step the last residual token is the new
// one, read from k_new / v_new.
template <int NQ, int WAVES = kWaves>
__device__ void residual_states(const AttnArgs& a, const RowState& rs, int64_t qrow0, int64_t kvrow, int wave,
                                float* o_dst, int o_stride, float (&mr)[NQ], float (&lr)[NQ]) {
    const int lane = threadIdx.x & 63, mrow = lane & 15, kq = lane >> 4;
    float o[NQ][2];
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        mr[r] = -INFINITY;
        lr[r] = 0.0f;
        o[r][0] = o[r][1] = 0.0f;
    }
    if (wave * kG >= rs.n_res) return;
    auto token_slot = [&](int i) { return (rs.res_head + i) % a.residual_cap; };
    auto is_new = [&](int i) { return a.k_new != nullptr && i == rs.n_res - 1; };
    // Memory round trips are what this phase waits on, so each chunk has one: the queries are
    // loaded once, first, then each chunk issues its key loads and all 32 value rows together
    // (a wave's loads complete in issue order, so the logits wait for the keys while the values
    // are still arriving).
    // Logits on the matrix cores (v_mfma_f32_16x16x32_f16, C = Q.K^T per 16-token tile): the A
    // operand's row m is query m (rows past NQ zero), the lane holding its channels
    // 32ks + 8kq .. +7 for each 32-channel step ks; the B operand's column n is the tile's token
    // n, whose 16 bytes of channels the lane loads from its row.  Query r's logit of token n
    // lands in lane n (< 16), accumulator entry r.
    uint4 qa[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qa[ks] = mrow < NQ ? *reinterpret_cast<const uint4*>(a.q + (qrow0 + mrow) * kD + 32 * ks + 8 * kq)
                           : make_uint4(0, 0, 0, 0);
    for (int base = wave * kG; base < rs.n_res; base += WAVES * kG) {
        const int nt = min(kG, rs.n_res - base);
        // ---- keys of tokens base + mrow and base + 16 + mrow, and the lane's two channels 2l,
        // 2l+1 of all the chunk's value rows (past the end: the chunk's first row again)
        uint4 kb[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int i = base + 16 * tt + mrow, j = i < rs.n_res ? i : base;
            const uint16_t* kr = is_new(j) ? a.k_new + kvrow * kD : a.k_res + (kvrow * a.residual_cap + token_slot(j)) * kD;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kb[tt][ks] = *reinterpret_cast<const uint4*>(kr + 32 * ks + 8 * kq);
        }
        uint32_t vv[kG];
#pragma unroll
        for (int u = 0; u < kG; ++u) {
            const int i = base + min(u, nt - 1);
            const uint16_t* row = is_new(i) ? a.v_new + kvrow * kD : a.v_res + (kvrow * a.residual_cap + token_slot(i)) * kD;
            vv[u] = reinterpret_cast<const uint32_t*>(row)[lane];
        }
        v4f acc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            acc[tt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, qa[ks]),
                                                                 __builtin_bit_cast(v8h, kb[tt][ks]), acc[tt], 0, 0, 0);
        }
        // ---- softmax over the chunk's tokens for every row (lanes 0..15: tokens mrow and
        // 16 + mrow; the reductions run over the lanes of the first 16-lane row)
        const bool ok0 = lane < 16 && base + mrow < rs.n_res, ok1 = lane < 16 && base + 16 + mrow < rs.n_res;
        _Float16* wts = reinterpret_cast<_Float16*>(o_dst);
        float al[NQ];
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            const float l0 = ok0 ? acc[0][r] * a.sm_log2 : -INFINITY, l1 = ok1 ? acc[1][r] * a.sm_log2 : -INFINITY;
            const float m_new = fmax_ieee(mr[r], readlane_f(row_max(fmax_ieee(l0, l1)), 0));
            al[r] = (mr[r] == -INFINITY) ? 0.0f : exp2_fast(mr[r] - m_new);
            const float p0 = ok0 ? exp2_fast(l0 - m_new) : 0.0f;
            const float p1 = ok1 ? exp2_fast(l1 - m_new) : 0.0f;
            lr[r] = lr[r] * al[r] + readlane_f(row_sum(p0 + p1), 0);
            mr[r] = m_new;
            // the weights as fp16, rounded to nearest (the quantized part's weights are fp16
            // too), at [row][token] of the scratch
            if (lane < 16) {
                wts[r * 2 * o_stride + mrow] = (_Float16)p0;
                wts[r * 2 * o_stride + 16 + mrow] = (_Float16)p1;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // ---- P.V: lane l takes channels 2l, 2l+1 of the chunk's token rows, two tokens per
        // packed dot product (tokens past the end carry weight 0)
#pragma unroll
        for (int r = 0; r < NQ; ++r) {
            o[r][0] *= al[r];
            o[r][1] *= al[r];
        }
#pragma unroll
        for (int t0 = 0; t0 < kG; t0 += 8) {
            if (t0 < nt) {
                // channel 2l of tokens t, t+1 in one register, channel 2l+1 in another
                uint32_t c0[4], c1[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    c0[u] = __builtin_amdgcn_perm(vv[t0 + 2 * u + 1], vv[t0 + 2 * u], 0x05040100u);
                    c1[u] = __builtin_amdgcn_perm(vv[t0 + 2 * u + 1], vv[t0 + 2 * u], 0x07060302u);
                }
#pragma unroll
                for (int r = 0; r < NQ; ++r) {
                    const uint4 pw = reinterpret_cast<const uint4*>(o_dst + r * o_stride)[t0 / 8];
                    const uint32_t pp[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        o[r][0] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, pp[u]), __builtin_bit_cast(h2v, c0[u]), o[r][0], false);
                        o[r][1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2v, pp[u]), __builtin_bit_cast(h2v, c1[u]), o[r][1], false);
                    }
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int r = 0; r < NQ; ++r) {
        o_dst[r * o_stride + 2 * lane] = o[r][0];
        o_dst[r * o_stride + 2 * lane + 1] = o[r][1];
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
// lse = (M + log2 L) ln 2.  A value whose tag is not this call's after the poll bound marks
// its row lost (sh_lost, cleared by the caller): the row's out and lse are written as NaN and
// the workspace status word gets kWsPollTimeout.  Re-arms the arrival counter and moves every
// row's epoch to this call's tag.
constexpr int kMergeBatch = 8;
template <int NQ, int THREADS = kBlock>
__device__ __forceinline__ void merge_rows(const AttnArgs& a, int splits, int64_t qrow0, uint32_t tag, int* sh_lost) {
    constexpr int kLpp = NQ == 1 ? THREADS / kD : 1;
    static_assert(NQ != 1 || (THREADS % kD == 0 && kLpp >= 2), "one row needs whole multiples of 128 threads");
    constexpr int kSweep = THREADS / kLpp;                  // (row, channel) pairs per pass
    constexpr int kIters = (NQ * kD + kSweep - 1) / kSweep;
    __shared__ float sh_mo[kLpp > 1 ? kLpp - 1 : 1][kD + 2];
    const int t = threadIdx.x, sub = kLpp > 1 ? t / kD : 0;
    const int64_t stride = a.q_rows * kPart;
    const uint32_t want = tag + a.tag_skew;                 // tag_skew: a test hook, 0 otherwise
    const int max_polls = a.max_polls > 0 ? a.max_polls : kMaxPolls;
    float Mi[kIters], Li[kIters], Oi[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int idx = (kLpp > 1 ? (t % kD) : t) + it * kSweep;
        Mi[it] = -INFINITY;
        Li[it] = Oi[it] = 0.0f;
        if (idx >= NQ * kD) continue;
        const int r = idx / kD, j = idx % kD;
        uint64_t* rowp = a.ws + (qrow0 + r) * kPart;
        bool lost = false;
        // a value of this call: loaded again until its tag is this call's, at most max_polls times
        auto settle = [&](uint64_t* p, uint64_t v) {
            for (int n = 0; (uint32_t)(v >> 32) != want && n < max_polls; ++n) {
                __builtin_amdgcn_s_sleep(1);
                v = load_coherent(p);
            }
            lost |= (uint32_t)(v >> 32) != want;
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
        if (lost) sh_lost[r] = 1;
        if (kLpp > 1 && sub > 0) {
            sh_mo[sub - 1][j] = O;
            if (j == 0) {
                sh_mo[sub - 1][kD] = M;
                sh_mo[sub - 1][kD + 1] = L;
            }
        }
        Mi[it] = M;
        Li[it] = L;
        Oi[it] = O;
    }
    __syncthreads();
    if (sub > 0) return;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        const int idx = (kLpp > 1 ? (t % kD) : t) + it * kSweep;
        if (idx >= NQ * kD) continue;
        const int r = idx / kD, j = idx % kD;
        float M = Mi[it], L = Li[it], O = Oi[it];
#pragma unroll
        for (int k = 0; k < kLpp - 1; ++k) {
            const float m1 = sh_mo[k][kD], l1 = sh_mo[k][kD + 1], o1 = sh_mo[k][j];
            const float mn = fmaxf(M, m1);
            const float al = M == -INFINITY ? 0.0f : exp2f(M - mn), be = m1 == -INFINITY ? 0.0f : exp2f(m1 - mn);
            L = fmaf(L, al, l1 * be);
            O = fmaf(O, al, o1 * be);
            M = mn;
        }
        const bool lost = sh_lost[r] != 0;
        a.out[(qrow0 + r) * kD + j] = lost ? 0x7E00u : (uint16_t)f2h(L > 0.0f ? O / L : 0.0f);
        if (j == 0 && a.lse != nullptr) a.lse[qrow0 + r] = lost ? __builtin_nanf("") : (M + log2f(L)) * 0.69314718055994531f;
    }
    if (t < NQ) {
        if (sh_lost[t]) __hip_atomic_fetch_or(a.status, kWsPollTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.counters[a.q_rows + qrow0 + t] = tag;   // the next call's partials for this row carry a larger tag
    }
    if (t == 0) a.counters[qrow0] = 0u;
}

// End of a WAVES-wave workgroup: merge its 2*WAVES states per row (empty states skipped), then write the
// output directly (one split) or the split partial, and let the last workgroup of the row
// group to arrive merge the partials.  Every partial value carries the call's tag (tag, from
// partial_tag at the workgroup's start), so the merging workgroup, which loads after its own
// arrival returned the final count, tells a value of this call from a stale one.  The
// arrival counter of a row group is the one of its first query row, in every kernel.
template <int NQ, int WAVES = kWaves>
__device__ __forceinline__ void finish_block(const AttnArgs& a, int splits, int split, int64_t qrow0, uint32_t tag, const float (*sh_o)[2 * WAVES][kD],
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
        arrived = __hip_atomic_fetch_add(&a.counters[qrow0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    __shared__ int sh_lost[NQ];
    if (threadIdx.x == kArrive) sh_last = arrived == (unsigned)(splits - 1);
    if (threadIdx.x < NQ) sh_lost[threadIdx.x] = 0;
    __syncthreads();
    if (sh_last) merge_rows<NQ, 64 * WAVES>(a, splits, qrow0, tag, sh_lost);
}

}  // namespace kivi
