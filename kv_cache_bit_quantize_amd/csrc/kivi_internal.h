// kivi_internal.h -- kernel argument blocks and launchers inside libkivi.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kivi {

constexpr int kMaxSplits = 1024;   // upper bound on split-K partitions of one decode call
constexpr int kCus = 256;          // compute units of the device (8 XCDs of 32)
constexpr int kSqWaves = 12;       // waves of a single-query attention workgroup (one per CU)
constexpr int kSqWavesMany = 4;    // ... for a uniform batch with more query rows than CUs (three per CU)

struct QuantArgs {          // kivi_quantize_{k,v}
    int32_t group;              // tokens per key group / channels per value group
    int32_t bits;               // code width: 2 or 4
    const uint16_t* src;
    int64_t src_row_stride;
    int64_t rows;
    int32_t tokens;
    int32_t dst_token_off;
    int32_t token_cap;
    uint8_t* k_codes;
    uint8_t* v_codes;
    uint16_t* k_sz;
    uint16_t* v_sz;
};

struct ResidualArgs {       // prefill: tokens [first, first+n) -> ring slots [0, n)
    const uint16_t* k;
    const uint16_t* v;
    int64_t src_row_stride;
    int64_t rows;
    int32_t first, n, residual_cap;
    uint16_t* k_res;
    uint16_t* v_res;
};

struct AppendArgs {
    const uint16_t* k_new;
    const uint16_t* v_new;
    int64_t rows;
    int32_t do_flush, flush_slot, flush_group, new_slot;
    int32_t token_cap, residual_cap;
    uint8_t* k_codes;
    uint8_t* v_codes;
    uint16_t* k_sz;
    uint16_t* v_sz;
    uint16_t* k_res;
    uint16_t* v_res;
    // ragged batch: per-sequence state [batch][4] (n_quant, n_res, res_head, flags) in device
    // memory; when set, every row takes its flush decision and slots from its sequence's
    // state instead of the fields above
    int32_t* seq_state;
    int32_t kv_heads;
    int32_t group;              // tokens per key group (= channels per value group): 32, 64 or 128
    int32_t flush_all;          // a flush moves the whole residual (else its oldest group)
    int32_t bits;               // code width: 2 or 4
    double rope_base;           // pre-RoPE keys (kivi_decode_attn_rope): the rotary base, else 0
    int32_t sq_waves;           // single-query 2-bit kernel: waves per workgroup (kSqWaves or kSqWavesMany)
};

struct AttnArgs {
    const uint16_t* q;          // [B][Hq][D]
    const uint8_t* k_codes;
    const uint8_t* v_codes;
    const uint16_t* k_sz;
    const uint16_t* v_sz;
    const uint16_t* k_res;
    const uint16_t* v_res;
    uint64_t* ws;               // [splits][B*Hq][D+2] partial (o, m, l), log2 domain: each value's bits
                                // in the low word, the call's tag in the high word
    uint32_t* counters;         // [B*Hq] arrival counters (zero between calls), then [B*Hq] call epochs
    uint32_t* status;           // the workspace's status word (bits ORed in: kWsPollTimeout)
    int32_t max_polls;          // polls of a partial before the merge gives up (0: the default bound)
    uint32_t tag_skew;          // test hook: the merge waits for tag + tag_skew (0 in every real call)
    uint16_t* out;              // [B][Hq][D]
    float* lse;                 // [B][Hq] or null
    float sm_log2;              // sm_scale * log2(e)
    int32_t q_heads, kv_heads, ratio;
    int32_t token_cap, residual_cap;
    int32_t n_quant, n_res, res_head;
    int32_t splits, groups_per_split;
    int64_t q_rows;             // B * Hq
    int32_t nq;                 // query heads per workgroup: 1, or 2..4 of one KV head's group
    int64_t block_rows;         // workgroup rows of the grid: B*Hq, or B*Hkv*(ratio/nq)
    // fused append (decode step): when k_new is set, residual token n_res - 1 is the new
    // token, read from k_new / v_new ([row][D]); one workgroup per KV row also writes it into
    // ring slot new_slot
    const uint16_t* k_new;
    const uint16_t* v_new;
    uint16_t* k_ring;           // k_res / v_res, written (the attention reads them as const)
    uint16_t* v_ring;
    int32_t new_slot;
    // fp16 comparator (kivi_decode_attn_fp16): keys and values [row][kv_stride][D] in fp16,
    // tokens [0, n_tokens) of each row valid, tokens_per_split of them per split
    const uint16_t* kf;
    const uint16_t* vf;
    int64_t kv_stride;
    int32_t n_tokens, tokens_per_split;
    // ragged batch: per-sequence state [batch][4] (n_quant, n_res, res_head, flags) in device
    // memory; when set it replaces n_quant, n_res, res_head and groups_per_split per row
    int32_t* seq_state;
    int32_t slot_budget;        // ragged batch: workgroups resident at once (the plan's target)
    int32_t group;              // tokens per key group (= channels per value group): 32, 64 or 128
    int32_t bits;               // code width: 2 or 4
    double rope_base;           // pre-RoPE keys (kivi_decode_attn_rope): the rotary base, else 0
    int32_t sq_waves;           // single-query 2-bit kernel: waves per workgroup (kSqWaves or kSqWavesMany)
};

// bits of a sequence's flags word (ragged calls; only ever set, by the kernels)
constexpr int32_t kSeqCapacity = 1;   // a flush would pass token_cap: the append was skipped
constexpr int32_t kSeqBadState = 2;   // the state was out of range: the sequence was skipped


// measurement helper: one streaming read of `bytes` (a multiple of 16) at src, plain loads or
// (streaming) non-temporal ones, one word per workgroup (kProbeBlocks of them) written to sink
constexpr int kProbeBlocks = 256;    // one 16-wave workgroup per CU
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, bool streaming, hipStream_t s,
                             hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

hipError_t launch_quantize_k(const QuantArgs& a, hipStream_t s);
hipError_t launch_quantize_v(const QuantArgs& a, hipStream_t s);
hipError_t launch_residual_load(const ResidualArgs& a, hipStream_t s);
hipError_t launch_append_flush(const AppendArgs& a, hipStream_t s);
// ragged append: the per-row appends, then the per-sequence state update
hipError_t launch_append_flush_ragged(const AppendArgs& a, int32_t batch, hipStream_t s);
// t0 / t1 (nullable): events that record the kernel's own start and end (hipExtLaunchKernel)
hipError_t launch_decode_attn(const AttnArgs& a, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_decode_attn_gqa(const AttnArgs& a, hipStream_t s, hipEvent_t t0 = nullptr,
                                  hipEvent_t t1 = nullptr);
hipError_t launch_decode_attn_rope(const AttnArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_decode_attn_q4(const AttnArgs& a, hipStream_t s, hipEvent_t t0 = nullptr,
                                 hipEvent_t t1 = nullptr);
hipError_t launch_decode_attn_fp16(const AttnArgs& a, hipStream_t s, hipEvent_t t0 = nullptr,
                                   hipEvent_t t1 = nullptr);

}  // namespace kivi
