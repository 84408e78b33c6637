// kivi_api.hip -- the extern "C" entry points of libkivi (declared in include/kivi.h).
//
// Every entry point validates its arguments on the host before it touches the HIP
// runtime, so the error paths run without a GPU.  Kernels are only enqueued on the
// caller's stream; nothing here allocates or synchronises.
#include "kivi.h"
#include "kivi_device.h"
#include "kivi_internal.h"

#include <cmath>
#include <mutex>

using namespace kivi;

// Scratch of kivi_decode_attn_noalloc: a workspace the library owns, one copy per device (the
// code object's static device memory), for callers that cannot allocate.  Host code takes its
// device address from hipGetSymbolAddress (per device, at the first call on that device) and
// never uses this name as an address.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
// zero n 16-byte words at p (the scratch's set-up, and its clearing when the shape changes)
__global__ void zero_words_kernel(uint4* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

// Per-device record of the scratch: its device address (0 until the first call on the device),
// the query-row count of the last call (the header and partial slots are laid out by it) and the
// high-water mark of the bytes any call has used.
struct NoAllocScratch {
    void* ptr = nullptr;
    int64_t q_rows = -1;
    size_t used = 0;
};
constexpr int kNoAllocDevices = 64;
std::mutex g_noalloc_mu;
NoAllocScratch g_noalloc[kNoAllocDevices];

}  // namespace

namespace {

// One round of resident workgroups on MI355X's 256 CUs: one 12-wave workgroup per CU for the
// single-query 2-bit kernel, 512 for the query-group kernel (measured best), three 4-wave
// workgroups per CU for the fp16 comparator.
constexpr int64_t kTargetBlocks = 768;         // 256-thread workgroups: three per CU
constexpr int64_t kTargetBlocksGroup = 512;    // query-group workgroups
constexpr int64_t kTargetBlocksSingle = 256;   // single-query 2-bit workgroups (12 waves): one per CU
constexpr int64_t kTargetBlocksQ4 = 1024;      // single-query 4-bit workgroups (4 waves): four per CU
// 4-bit query-group workgroups (four query heads, 106 VGPRs): two rounds of four per CU.  On
// gqa-mistral-7b (512 kv rows) one split took 233 us, 2 / 4 / 6 / 8 splits 194-205 / 183-199 /
// 189-203 / 200 us on two GPUs, 12 splits 234 us
constexpr int64_t kTargetBlocksQ4Group = 2048;
constexpr int kMinGroupsPerSplit = 8;
constexpr int kMinGroupsPerSplitSingle = 2 * kSqWaves;   // a pair of tiles for every wave

constexpr int32_t kMaxTokenCap4 = 1 << 26;
constexpr int32_t kMaxTokenCapRope2 = 1 << 27;   // 2-bit rows under 32-bit byte offsets (pre-RoPE kernel)
constexpr int64_t kWavesRope = 4;
constexpr int64_t kTargetBlocksRope = 768;
constexpr int64_t kTargetBlocksRopeGroup = 512;   // query-group form: two workgroups per CU

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const kivi_cache* c) {
    if (c == nullptr) return KIVI_ERR_NULL;
    if (c->batch <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 || c->group <= 0 ||
        c->residual_cap <= 0 || c->token_cap < 0 || (c->flags & ~(KIVI_FLUSH_ALL | KIVI_CODES_4BIT)) != 0)
        return KIVI_ERR_SHAPE;
    if (c->head_dim % 4 != 0 || c->head_dim % c->group != 0 || c->residual_cap % c->group != 0 ||
        c->token_cap % c->group != 0)
        return KIVI_ERR_SHAPE;
    if (c->head_dim != kD || !group_supported(c->group)) return KIVI_ERR_UNSUPPORTED;
    // 4-bit rows are addressed with 32-bit byte offsets: token_cap * 64 < 2^32
    if ((c->flags & KIVI_CODES_4BIT) && c->token_cap > kMaxTokenCap4) return KIVI_ERR_UNSUPPORTED;
    return KIVI_OK;
}

int check_state(const kivi_cache* c) {
    const int G = c->group, R = c->residual_cap;
    if (c->n_quant < 0 || c->n_quant % G != 0 || c->n_quant > c->token_cap) return KIVI_ERR_STATE;
    if (c->n_res < 0 || c->n_res > R) return KIVI_ERR_STATE;
    if (c->res_head < 0 || c->res_head >= R || c->res_head % G != 0) return KIVI_ERR_STATE;
    return KIVI_OK;
}

int check_quant_bufs(const kivi_cache* c, bool keys, bool values) {
    if (keys && (c->k_codes == nullptr || c->k_sz == nullptr)) return KIVI_ERR_NULL;
    if (values && (c->v_codes == nullptr || c->v_sz == nullptr)) return KIVI_ERR_NULL;
    if (keys && (!aligned16(c->k_codes) || !aligned16(c->k_sz))) return KIVI_ERR_SHAPE;
    if (values && (!aligned16(c->v_codes) || !aligned16(c->v_sz))) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

int check_res_bufs(const kivi_cache* c) {
    if (c->k_res == nullptr || c->v_res == nullptr) return KIVI_ERR_NULL;
    if (!aligned16(c->k_res) || !aligned16(c->v_res)) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

int64_t rows_of(const kivi_cache* c) { return (int64_t)c->batch * c->kv_heads; }

int hip_status(hipError_t e) { return e == hipSuccess ? KIVI_OK : KIVI_ERR_HIP; }

// Query heads one workgroup takes: a KV head's query group (or an equal share of it) goes
// to one workgroup, which streams the KV head's cache once for all of them.
int32_t code_bits(const kivi_cache* c) { return (c->flags & KIVI_CODES_4BIT) ? 4 : 2; }

// query heads per workgroup for a GQA ratio (the 4-bit kernel: one, two or four; with four
// heads it needs 106 VGPRs, and a kv head's four query heads in one workgroup read its codes
// once: gqa-mistral-7b 233 us against 245-251 us with two heads per workgroup)
int32_t queries_per_block(int32_t ratio, int32_t bits = 2) {
    if (bits == 4) return ratio % 4 == 0 ? 4 : (ratio % 2 == 0 ? 2 : 1);
    if (ratio % 4 == 0) return 4;
    if (ratio % 3 == 0) return 3;
    if (ratio % 2 == 0) return 2;
    return 1;
}

// workgroup rows of the attention grid
int64_t block_rows(const kivi_cache* c, int32_t q_heads) {
    const int32_t ratio = q_heads / c->kv_heads;
    const int32_t nq = queries_per_block(ratio, code_bits(c));
    return nq > 1 ? (int64_t)c->batch * c->kv_heads * (ratio / nq) : (int64_t)c->batch * q_heads;
}

// Waves per workgroup of the single-query 2-bit kernel for a uniform batch: one 12-wave
// workgroup per CU when the query rows are no more than the CUs (the rows are split across
// them), else 4-wave workgroups, three per CU, so that up to 768 rows run in one round.
int32_t single_query_waves(const kivi_cache* c, int32_t q_heads) {
    const bool single = code_bits(c) == 2 && queries_per_block(q_heads / c->kv_heads) == 1;
    return single && (int64_t)c->batch * q_heads > kTargetBlocksSingle ? kSqWavesMany : kSqWaves;
}

// Split count for a context of `groups` key groups (waves: the single-query kernel's).
int32_t auto_splits_for(const kivi_cache* c, int32_t q_heads, int64_t groups, int32_t waves = kSqWaves) {
    const int64_t rows = block_rows(c, q_heads);
    const bool group = queries_per_block(q_heads / c->kv_heads, code_bits(c)) > 1;
    int64_t target = group ? kTargetBlocksGroup : kTargetBlocksSingle;
    int64_t min_tiles = group ? kMinGroupsPerSplit : kMinGroupsPerSplitSingle;
    if (!group && code_bits(c) == 2 && waves == kSqWavesMany) {
        // three workgroups per CU, a pair of tiles for every wave; as many splits as keep the
        // call within one round (the rows alone already fill a round at 384 rows and more)
        int64_t s = kTargetBlocks / rows;
        const int64_t cap = groups / (2 * kSqWavesMany);
        if (s > cap) s = cap;
        return (int32_t)(s < 1 ? 1 : s);
    }
    if (code_bits(c) == 4) {   // 4-wave workgroups, a key group for every wave
        // one query head: four workgroups per CU (88 VGPRs; at 131,072 tokens 32 splits took
        // 124-128 us against 129-146 us for 24 on three GPUs)
        target = group ? kTargetBlocksQ4Group : kTargetBlocksQ4;
        min_tiles = 4 * (c->group / kG);
    }
    int64_t s = (target + rows - 1) / rows;
    const int64_t cap = groups / min_tiles;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int32_t)s;
}
// (contexts are counted in 32-token code tiles, the attention kernels' unit of work)
int32_t auto_splits(const kivi_cache* c, int32_t q_heads) {
    return auto_splits_for(c, q_heads, c->n_quant / kG, single_query_waves(c, q_heads));
}
// ragged batch: room for four times the splits of the longest context the cache can hold;
// the kernels plan from the real lengths how many of them each sequence uses
int32_t ragged_auto_splits(const kivi_cache* c, int32_t q_heads) {
    const int64_t groups = c->token_cap / kG;
    int64_t s = 4 * (int64_t)auto_splits_for(c, q_heads, groups);
    const bool group = queries_per_block(q_heads / c->kv_heads, code_bits(c)) > 1;
    const int64_t min_tiles = code_bits(c) == 4 ? 4 * (c->group / kG) : (group ? kMinGroupsPerSplit : kMinGroupsPerSplitSingle);
    const int64_t cap = groups / min_tiles;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int32_t)s;
}

// Leading area of an attention workspace: the status word in a 256-byte block of its own, then
// one arrival counter per query row and one call epoch per query row (the tag of the last
// partials merged for that row), rounded up to 256 bytes.
constexpr size_t kStatusBytes = 256;
size_t header_bytes(int64_t q_rows) {
    return kStatusBytes + ((2 * (size_t)q_rows * sizeof(uint32_t) + 255) & ~(size_t)255);
}
size_t counter_bytes(const kivi_cache* c, int32_t q_heads) { return header_bytes((int64_t)c->batch * q_heads); }

// Test hook of the merge's bounded wait (kivi_test_next_attention_merge): consumed by the next
// attention call of this thread that passes validation.
thread_local int32_t t_merge_polls = 0;
thread_local uint32_t t_merge_skew = 0;
void take_merge_test(AttnArgs* a) {
    a->max_polls = t_merge_polls;
    a->tag_skew = t_merge_skew;
    t_merge_polls = 0;
    t_merge_skew = 0;
}
// Header pointers of a workspace
void set_header(AttnArgs* a, void* workspace, size_t header) {
    a->status = static_cast<uint32_t*>(workspace);
    a->counters = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kStatusBytes);
    a->ws = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + header);
}

QuantArgs quant_args(const kivi_cache* c, const uint16_t* src, int32_t tokens, int64_t stride,
                     int32_t dst) {
    QuantArgs a;
    a.src = src;
    a.src_row_stride = stride;
    a.rows = rows_of(c);
    a.tokens = tokens;
    a.dst_token_off = dst;
    a.token_cap = c->token_cap;
    a.k_codes = c->k_codes;
    a.v_codes = c->v_codes;
    a.k_sz = c->k_sz;
    a.v_sz = c->v_sz;
    a.group = c->group;
    a.bits = code_bits(c);
    return a;
}

// The state after one append (record "KV bytes basis": the newest R tokens stay in 16-bit
// floats, only grouped history is quantized): a full ring first gives its oldest F tokens
// (F = G, or R with KIVI_FLUSH_ALL) to the history, then the new token enters the ring.
// *flush tells whether a flush happens.  Expects a valid shape and state.
int post_append_state(const kivi_cache* c, kivi_cache* next, bool* flush) {
    const int G = c->group, R = c->residual_cap;
    const int F = (c->flags & KIVI_FLUSH_ALL) ? R : G;   // tokens a flush moves
    *flush = c->n_res == R;
    if (*flush && c->n_quant + F > c->token_cap) return KIVI_ERR_CAPACITY;
    *next = *c;
    if (*flush) {
        next->n_quant += F;
        next->res_head = (c->res_head + F) % R;
        next->n_res -= F;
    }
    next->n_res += 1;
    return KIVI_OK;
}

// Validates an append and fills its arguments; *next receives the state after it.
int prepare_append(const kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new, AppendArgs* a,
                   kivi_cache* next) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_state(c)) != KIVI_OK) return st;
    if ((st = check_quant_bufs(c, true, true)) != KIVI_OK) return st;
    if ((st = check_res_bufs(c)) != KIVI_OK) return st;
    if (k_new == nullptr || v_new == nullptr) return KIVI_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_ERR_SHAPE;
    const int G = c->group, R = c->residual_cap;
    bool flush = false;
    if ((st = post_append_state(c, next, &flush)) != KIVI_OK) return st;
    a->k_new = k_new;
    a->v_new = v_new;
    a->rows = rows_of(c);
    a->do_flush = flush ? 1 : 0;
    a->flush_slot = c->res_head;
    a->flush_group = c->n_quant / G;
    a->new_slot = (next->res_head + next->n_res - 1) % R;
    a->token_cap = c->token_cap;
    a->residual_cap = R;
    a->k_codes = c->k_codes;
    a->v_codes = c->v_codes;
    a->k_sz = c->k_sz;
    a->v_sz = c->v_sz;
    a->k_res = c->k_res;
    a->v_res = c->v_res;
    a->seq_state = nullptr;   // one state for the whole batch (the fields above)
    a->kv_heads = c->kv_heads;
    a->group = G;
    a->flush_all = (c->flags & KIVI_FLUSH_ALL) ? 1 : 0;
    a->bits = code_bits(c);
    return KIVI_OK;
}

void commit_state(kivi_cache* c, const kivi_cache& next) {
    c->n_quant = next.n_quant;
    c->n_res = next.n_res;
    c->res_head = next.res_head;
}

// Pre-RoPE attention: one query head per 4-wave workgroup, a key group for every wave, and
// one round of three workgroups per CU (the kernel's 157-164 VGPRs leave room for three; at
// 131,072 tokens and 32 heads 24 splits took 168 us, 16 splits 201 us, 32 splits 190 us).
// With a GQA ratio divisible by two or three a kv head's query heads share a workgroup, four,
// three or two of them (rope_queries_per_block), which turns each key once for all of them; at
// 180-256 VGPRs two such workgroups fit per CU, and one round of them is the target
// (gqa-mistral-7b: one split, 224-265 us, against 247-275 us for two and 279-301 us for three
// or four).
int32_t rope_queries_per_block(const kivi_cache* c, int32_t q_heads) {
    const int32_t ratio = q_heads / c->kv_heads;
    return ratio % 4 == 0 ? 4 : (ratio % 3 == 0 ? 3 : (ratio % 2 == 0 ? 2 : 1));
}
int32_t rope_splits_for(const kivi_cache* c, int32_t q_heads, int64_t groups) {
    const int32_t nq = rope_queries_per_block(c, q_heads);
    const int64_t rows = (int64_t)c->batch * q_heads / nq;
    const int64_t target = nq > 1 ? kTargetBlocksRopeGroup : kTargetBlocksRope;
    int64_t s = (target + rows - 1) / rows;
    if (s > groups / kWavesRope) s = groups / kWavesRope;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int32_t)s;
}
int32_t rope_auto_splits(const kivi_cache* c, int32_t q_heads) { return rope_splits_for(c, q_heads, c->n_quant / c->group); }
// ragged batch: room for four times the splits of the longest context the cache can hold
int32_t rope_ragged_splits(const kivi_cache* c, int32_t q_heads) {
    const int64_t groups = c->token_cap / c->group;
    int64_t s = 4 * (int64_t)rope_splits_for(c, q_heads, groups);
    if (s > groups / kWavesRope) s = groups / kWavesRope;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int32_t)s;
}

// Validates a decode-attention call on cache state *c (or, with seq_state, on the
// per-sequence device states of a ragged batch, which the kernels check) and fills its
// arguments.
int prepare_attn(const kivi_cache* c, const uint16_t* q, int32_t q_heads, float sm_scale, uint16_t* out,
                 float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits, AttnArgs* pa,
                 int32_t* seq_state = nullptr) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if (seq_state == nullptr && (st = check_state(c)) != KIVI_OK) return st;
    if (seq_state != nullptr && !aligned16(seq_state)) return KIVI_ERR_SHAPE;
    if ((st = check_quant_bufs(c, true, true)) != KIVI_OK) return st;
    if ((st = check_res_bufs(c)) != KIVI_OK) return st;
    if (q == nullptr || out == nullptr) return KIVI_ERR_NULL;
    if (!aligned16(q) || (reinterpret_cast<uintptr_t>(out) & 1u) || (reinterpret_cast<uintptr_t>(lse) & 3u))
        return KIVI_ERR_SHAPE;
    if (q_heads <= 0 || q_heads % c->kv_heads != 0) return KIVI_ERR_SHAPE;
    if (seq_state == nullptr && c->n_quant + c->n_res == 0) return KIVI_ERR_SHAPE;
    if (num_splits < 0 || num_splits > kMaxSplits) return KIVI_ERR_SHAPE;
    if (!std::isfinite(sm_scale)) return KIVI_ERR_SHAPE;
    const int32_t splits =
        num_splits > 0 ? num_splits : (seq_state != nullptr ? ragged_auto_splits(c, q_heads) : auto_splits(c, q_heads));
    const size_t need = kivi_decode_attn_workspace(c, q_heads, splits);
    if (workspace == nullptr || workspace_bytes < need) return KIVI_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return KIVI_ERR_WORKSPACE;
    const int32_t groups = c->n_quant / kG;   // 32-token code tiles
    AttnArgs a{};
    a.q = q;
    a.k_codes = c->k_codes;
    a.v_codes = c->v_codes;
    a.k_sz = c->k_sz;
    a.v_sz = c->v_sz;
    a.k_res = c->k_res;
    a.v_res = c->v_res;
    set_header(&a, workspace, counter_bytes(c, q_heads));
    a.out = out;
    a.lse = lse;
    a.sm_log2 = (float)((double)sm_scale * 1.4426950408889634);
    a.q_heads = q_heads;
    a.kv_heads = c->kv_heads;
    a.ratio = q_heads / c->kv_heads;
    a.token_cap = c->token_cap;
    a.residual_cap = c->residual_cap;
    a.n_quant = c->n_quant;
    a.n_res = c->n_res;
    a.res_head = c->res_head;
    a.splits = splits;
    // The last split also reads the fp16 residual (512 bytes per token against 96 for a
    // quantized token): count it as that many groups so the last split gets fewer.
    const int32_t res_groups = (c->n_res * 512 + 96 * kG - 1) / (96 * kG);
    a.groups_per_split = (groups + res_groups + splits - 1) / splits;
    a.q_rows = (int64_t)c->batch * q_heads;
    a.nq = queries_per_block(a.ratio, code_bits(c));
    a.block_rows = block_rows(c, q_heads);
    a.k_new = a.v_new = nullptr;
    a.k_ring = a.v_ring = nullptr;
    a.new_slot = 0;
    a.seq_state = seq_state;
    // workgroups resident at once: three 4-wave query-group workgroups or one 12-wave
    // single-query workgroup per CU
    a.slot_budget = (int32_t)(a.nq > 1 || code_bits(c) == 4 ? kTargetBlocks : kTargetBlocksSingle);
    // the ragged plan counts query rows in 32 bits (and launches them in one grid dimension)
    if (seq_state != nullptr && a.q_rows > INT32_MAX) return KIVI_ERR_SHAPE;
    a.group = c->group;
    a.bits = code_bits(c);
    // ragged batches keep one 12-wave workgroup per CU (their plan shares a round of 256)
    a.sq_waves = seq_state == nullptr ? single_query_waves(c, q_heads) : kSqWaves;
    take_merge_test(&a);
    *pa = a;
    return KIVI_OK;
}

// ---- fp16 comparator
constexpr int kMinTokensPerSplit = 256;

int64_t fp16_block_rows(int32_t batch, int32_t kv_heads, int32_t q_heads) {
    const int32_t ratio = q_heads / kv_heads;
    const int32_t nq = queries_per_block(ratio);
    return nq > 1 ? (int64_t)batch * kv_heads * (ratio / nq) : (int64_t)batch * q_heads;
}

int fp16_check(int32_t batch, int32_t kv_heads, int32_t tokens, int32_t q_heads) {
    if (batch <= 0 || kv_heads <= 0 || q_heads <= 0 || q_heads % kv_heads != 0) return KIVI_ERR_SHAPE;
    if (tokens <= 0) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

int32_t fp16_auto_splits(int32_t batch, int32_t kv_heads, int32_t tokens, int32_t q_heads) {
    const int64_t rows = fp16_block_rows(batch, kv_heads, q_heads);
    const int64_t target = queries_per_block(q_heads / kv_heads) > 1 ? kTargetBlocksGroup : kTargetBlocks;
    int64_t s = (target + rows - 1) / rows;
    const int64_t cap = tokens / kMinTokensPerSplit;
    if (s > cap) s = cap;
    if (s < 1) s = 1;
    if (s > kMaxSplits) s = kMaxSplits;
    return (int32_t)s;
}

size_t fp16_counter_bytes(int32_t batch, int32_t q_heads) { return header_bytes((int64_t)batch * q_heads); }

// Events for the next attention launch of this thread (kivi_time_next_attention).
thread_local hipEvent_t t_timing[2] = {nullptr, nullptr};
void take_timing(hipEvent_t* t0, hipEvent_t* t1) {
    *t0 = t_timing[0];
    *t1 = t_timing[1];
    t_timing[0] = t_timing[1] = nullptr;
}

}  // namespace

extern "C" {

const char* kivi_status_str(int status) {
    switch (status) {
        case KIVI_OK: return "ok";
        case KIVI_ERR_NULL: return "a required pointer is NULL";
        case KIVI_ERR_SHAPE: return "inconsistent sizes, strides or alignment";
        case KIVI_ERR_UNSUPPORTED: return "shape not implemented (head_dim must be 128, group 32, 64 or 128)";
        case KIVI_ERR_CAPACITY: return "the call would write past token_cap";
        case KIVI_ERR_WORKSPACE: return "workspace missing or too small";
        case KIVI_ERR_HIP: return "HIP runtime error while enqueueing";
        case KIVI_ERR_STATE: return "inconsistent cache state (n_quant, n_res, res_head)";
        default: return "unknown status";
    }
}

int kivi_cache_bytes(const kivi_cache* shape, size_t* codes, size_t* pairs, size_t* residual) {
    int st = check_shape(shape);
    if (st != KIVI_OK) return st;
    if (codes == nullptr || pairs == nullptr || residual == nullptr) return KIVI_ERR_NULL;
    const int64_t rows = rows_of(shape), D = shape->head_dim, G = shape->group;
    const int64_t T = shape->token_cap, R = shape->residual_cap;
    *codes = (size_t)(2 * rows * T * (D * code_bits(shape) / 8));
    *pairs = (size_t)(rows * (T / G) * D * 4 + rows * T * (D / G) * 4);
    *residual = (size_t)(2 * rows * R * D * 2);
    return KIVI_OK;
}

int kivi_quantize_k_per_channel(const uint16_t* k, int32_t tokens, int64_t src_row_stride,
                                kivi_cache* c, int32_t dst_token_off, void* stream) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_quant_bufs(c, true, false)) != KIVI_OK) return st;
    if (tokens < 0 || dst_token_off < 0 || tokens % c->group != 0 || dst_token_off % c->group != 0)
        return KIVI_ERR_SHAPE;
    if ((int64_t)dst_token_off + tokens > c->token_cap) return KIVI_ERR_CAPACITY;
    if (tokens == 0) return KIVI_OK;
    if (k == nullptr) return KIVI_ERR_NULL;
    if (src_row_stride < (int64_t)tokens * c->head_dim || src_row_stride % 8 != 0 || !aligned16(k))
        return KIVI_ERR_SHAPE;
    return hip_status(launch_quantize_k(quant_args(c, k, tokens, src_row_stride, dst_token_off),
                                        (hipStream_t)stream));
}

int kivi_quantize_v_per_token(const uint16_t* v, int32_t tokens, int64_t src_row_stride,
                              kivi_cache* c, int32_t dst_token_off, void* stream) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_quant_bufs(c, false, true)) != KIVI_OK) return st;
    if (tokens < 0 || dst_token_off < 0) return KIVI_ERR_SHAPE;
    if ((int64_t)dst_token_off + tokens > c->token_cap) return KIVI_ERR_CAPACITY;
    if (tokens == 0) return KIVI_OK;
    if (v == nullptr) return KIVI_ERR_NULL;
    if (src_row_stride < (int64_t)tokens * c->head_dim || src_row_stride % 8 != 0 || !aligned16(v))
        return KIVI_ERR_SHAPE;
    return hip_status(launch_quantize_v(quant_args(c, v, tokens, src_row_stride, dst_token_off),
                                        (hipStream_t)stream));
}

int kivi_prefill(const uint16_t* k, const uint16_t* v, int32_t tokens, int64_t src_row_stride,
                 int32_t n_quant, kivi_cache* c, void* stream) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_quant_bufs(c, true, true)) != KIVI_OK) return st;
    if ((st = check_res_bufs(c)) != KIVI_OK) return st;
    if (tokens < 0 || n_quant < 0 || n_quant > tokens || n_quant % c->group != 0) return KIVI_ERR_SHAPE;
    if (n_quant > c->token_cap || tokens - n_quant > c->residual_cap) return KIVI_ERR_CAPACITY;
    if (tokens > 0) {
        if (k == nullptr || v == nullptr) return KIVI_ERR_NULL;
        if (src_row_stride < (int64_t)tokens * c->head_dim || src_row_stride % 8 != 0 || !aligned16(k) ||
            !aligned16(v))
            return KIVI_ERR_SHAPE;
    }
    hipStream_t s = (hipStream_t)stream;
    if (n_quant > 0) {
        if ((st = hip_status(launch_quantize_k(quant_args(c, k, n_quant, src_row_stride, 0), s))) != KIVI_OK)
            return st;
        if ((st = hip_status(launch_quantize_v(quant_args(c, v, n_quant, src_row_stride, 0), s))) != KIVI_OK)
            return st;
    }
    if (tokens > n_quant) {
        ResidualArgs r;
        r.k = k;
        r.v = v;
        r.src_row_stride = src_row_stride;
        r.rows = rows_of(c);
        r.first = n_quant;
        r.n = tokens - n_quant;
        r.residual_cap = c->residual_cap;
        r.k_res = c->k_res;
        r.v_res = c->v_res;
        if ((st = hip_status(launch_residual_load(r, s))) != KIVI_OK) return st;
    }
    c->n_quant = n_quant;
    c->n_res = tokens - n_quant;
    c->res_head = 0;
    return KIVI_OK;
}

int kivi_append_flush(kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new, int32_t* flushed,
                      void* stream) {
    AppendArgs a;
    kivi_cache next;
    int st = prepare_append(c, k_new, v_new, &a, &next);
    if (st != KIVI_OK) return st;
    if ((st = hip_status(launch_append_flush(a, (hipStream_t)stream))) != KIVI_OK) return st;
    commit_state(c, next);
    if (flushed != nullptr) *flushed = a.do_flush;
    return KIVI_OK;
}

int kivi_append_flush_ragged(const kivi_cache* c, int32_t* seq_state, const uint16_t* k_new, const uint16_t* v_new,
                             void* stream) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_quant_bufs(c, true, true)) != KIVI_OK) return st;
    if ((st = check_res_bufs(c)) != KIVI_OK) return st;
    if (seq_state == nullptr || k_new == nullptr || v_new == nullptr) return KIVI_ERR_NULL;
    if (!aligned16(seq_state) || !aligned16(k_new) || !aligned16(v_new)) return KIVI_ERR_SHAPE;
    AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.rows = rows_of(c);
    a.token_cap = c->token_cap;
    a.residual_cap = c->residual_cap;
    a.k_codes = c->k_codes;
    a.v_codes = c->v_codes;
    a.k_sz = c->k_sz;
    a.v_sz = c->v_sz;
    a.k_res = c->k_res;
    a.v_res = c->v_res;
    a.seq_state = seq_state;
    a.kv_heads = c->kv_heads;
    a.group = c->group;
    a.flush_all = (c->flags & KIVI_FLUSH_ALL) ? 1 : 0;
    a.bits = code_bits(c);
    return hip_status(launch_append_flush_ragged(a, c->batch, (hipStream_t)stream));
}

int kivi_decode_attn_ragged(const kivi_cache* c, int32_t* seq_state, const uint16_t* q, int32_t q_heads,
                            float sm_scale, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                            int32_t num_splits, void* stream) {
    if (seq_state == nullptr) return KIVI_ERR_NULL;
    AttnArgs a;
    const int st =
        prepare_attn(c, q, q_heads, sm_scale, out, lse, workspace, workspace_bytes, num_splits, &a, seq_state);
    if (st != KIVI_OK) return st;
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    return hip_status(launch_decode_attn(a, (hipStream_t)stream, t0, t1));
}

int32_t kivi_decode_attn_ragged_splits(const kivi_cache* c, int32_t q_heads) {
    const int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if (q_heads <= 0 || q_heads % c->kv_heads != 0) return KIVI_ERR_SHAPE;
    return ragged_auto_splits(c, q_heads);
}

int32_t kivi_decode_attn_splits(const kivi_cache* c, int32_t q_heads) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_state(c)) != KIVI_OK) return st;
    if (q_heads <= 0 || q_heads % c->kv_heads != 0) return KIVI_ERR_SHAPE;
    return auto_splits(c, q_heads);
}

size_t kivi_decode_attn_workspace(const kivi_cache* c, int32_t q_heads, int32_t num_splits) {
    if (check_shape(c) != KIVI_OK || q_heads <= 0) return 0;
    const int32_t s = num_splits > 0 ? num_splits : auto_splits(c, q_heads);
    const size_t bytes = (size_t)s * (size_t)c->batch * (size_t)q_heads * (size_t)(c->head_dim + 2) * sizeof(uint64_t);
    return counter_bytes(c, q_heads) + ((bytes + 255) & ~(size_t)255);
}

int32_t kivi_decode_attn_fp16_splits(int32_t batch, int32_t kv_heads, int32_t tokens, int32_t q_heads) {
    const int st = fp16_check(batch, kv_heads, tokens, q_heads);
    if (st != KIVI_OK) return st;
    return fp16_auto_splits(batch, kv_heads, tokens, q_heads);
}

size_t kivi_decode_attn_fp16_workspace(int32_t batch, int32_t kv_heads, int32_t tokens, int32_t q_heads,
                                       int32_t num_splits) {
    if (fp16_check(batch, kv_heads, tokens, q_heads) != KIVI_OK || num_splits < 0) return 0;
    const int32_t s = num_splits > 0 ? num_splits : fp16_auto_splits(batch, kv_heads, tokens, q_heads);
    const size_t bytes = (size_t)s * (size_t)batch * (size_t)q_heads * (size_t)(kD + 2) * sizeof(uint64_t);
    return fp16_counter_bytes(batch, q_heads) + ((bytes + 255) & ~(size_t)255);
}

int kivi_decode_attn_fp16(const uint16_t* k, const uint16_t* v, int32_t batch, int32_t kv_heads, int32_t tokens,
                          int32_t token_stride, const uint16_t* q, int32_t q_heads, float sm_scale, uint16_t* out,
                          float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits, void* stream) {
    if (k == nullptr || v == nullptr || q == nullptr || out == nullptr) return KIVI_ERR_NULL;
    int st = fp16_check(batch, kv_heads, tokens, q_heads);
    if (st != KIVI_OK) return st;
    if (token_stride < tokens) return KIVI_ERR_SHAPE;
    if (!aligned16(k) || !aligned16(v) || !aligned16(q) || (reinterpret_cast<uintptr_t>(out) & 1u) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return KIVI_ERR_SHAPE;
    if (num_splits < 0 || num_splits > kMaxSplits) return KIVI_ERR_SHAPE;
    if (!std::isfinite(sm_scale)) return KIVI_ERR_SHAPE;
    const int32_t splits = num_splits > 0 ? num_splits : fp16_auto_splits(batch, kv_heads, tokens, q_heads);
    const size_t need = kivi_decode_attn_fp16_workspace(batch, kv_heads, tokens, q_heads, splits);
    if (workspace == nullptr || workspace_bytes < need) return KIVI_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return KIVI_ERR_WORKSPACE;
    AttnArgs a{};
    a.q = q;
    set_header(&a, workspace, fp16_counter_bytes(batch, q_heads));
    a.out = out;
    a.lse = lse;
    a.sm_log2 = (float)((double)sm_scale * 1.4426950408889634);
    a.q_heads = q_heads;
    a.kv_heads = kv_heads;
    a.ratio = q_heads / kv_heads;
    a.splits = splits;
    a.q_rows = (int64_t)batch * q_heads;
    a.nq = queries_per_block(a.ratio);
    a.block_rows = fp16_block_rows(batch, kv_heads, q_heads);
    a.kf = k;
    a.vf = v;
    a.kv_stride = token_stride;
    a.n_tokens = tokens;
    a.tokens_per_split = (tokens + splits - 1) / splits;
    take_merge_test(&a);
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    return hip_status(launch_decode_attn_fp16(a, (hipStream_t)stream, t0, t1));
}

int kivi_test_next_attention_merge(int32_t max_polls, uint32_t tag_skew) {
    if (max_polls < 0) return KIVI_ERR_SHAPE;
    t_merge_polls = max_polls;
    t_merge_skew = tag_skew;
    return KIVI_OK;
}

size_t kivi_read_probe_sink_bytes(void) { return (size_t)kProbeBlocks * sizeof(uint32_t); }

static int read_probe(const void* src, size_t bytes, uint32_t* sink, bool streaming, void* stream) {
    if (src == nullptr || sink == nullptr) return KIVI_ERR_NULL;
    if (bytes % 16 != 0 || !aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return KIVI_ERR_SHAPE;
    if (bytes == 0) return KIVI_OK;
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    return hip_status(launch_read_probe(src, bytes, sink, streaming, (hipStream_t)stream, t0, t1));
}

int kivi_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    return read_probe(src, bytes, sink, false, stream);
}

int kivi_read_probe_stream(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    return read_probe(src, bytes, sink, true, stream);
}

int kivi_time_next_attention(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return KIVI_ERR_NULL;
    t_timing[0] = static_cast<hipEvent_t>(start_event);
    t_timing[1] = static_cast<hipEvent_t>(stop_event);
    return KIVI_OK;
}

int kivi_decode_attn_noalloc(const kivi_cache* c, const uint16_t* q, int32_t q_heads, float sm_scale, uint16_t* out,
                             float* lse, int32_t num_splits, void* stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KIVI_ERR_HIP;
    if (dev < 0 || dev >= kNoAllocDevices) return KIVI_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    NoAllocScratch& sc = g_noalloc[dev];
    if (sc.ptr == nullptr) {   // set-up on this device, with it current
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KIVI_ERR_HIP;
        sc.ptr = p;
        sc.q_rows = -1;
        sc.used = kNoAllocScratchBytes;   // cleared whole before the first call uses it
    }
    AttnArgs a;
    // validation, split count and the size check (KIVI_ERR_WORKSPACE beyond the scratch's size)
    int st = prepare_attn(c, q, q_heads, sm_scale, out, lse, sc.ptr, kNoAllocScratchBytes, num_splits, &a);
    if (st != KIVI_OK) return st;
    const size_t need = kivi_decode_attn_workspace(c, q_heads, a.splits);
    hipStream_t s = (hipStream_t)stream;
    if (sc.q_rows != a.q_rows) {
        // another shape: the counters, epochs and partial slots move, so everything any call has
        // written is cleared first (same stream, before the attention); with an unchanged shape the
        // scratch stays consistent from call to call, as a workspace does
        const size_t bytes = sc.used > need ? sc.used : need;
        const size_t words = bytes / 16;
        const unsigned blocks = (unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024);
        hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint4*>(sc.ptr), words);
        if ((st = hip_status(hipGetLastError())) != KIVI_OK) return st;
        sc.q_rows = a.q_rows;
        sc.used = need;
    } else if (need > sc.used) {
        sc.used = need;
    }
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    return hip_status(launch_decode_attn(a, s, t0, t1));
}

int kivi_decode_attn(const kivi_cache* c, const uint16_t* q, int32_t q_heads, float sm_scale, uint16_t* out,
                     float* lse, void* workspace, size_t workspace_bytes, int32_t num_splits, void* stream) {
    AttnArgs a;
    const int st = prepare_attn(c, q, q_heads, sm_scale, out, lse, workspace, workspace_bytes, num_splits, &a);
    if (st != KIVI_OK) return st;
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    return hip_status(launch_decode_attn(a, (hipStream_t)stream, t0, t1));
}

// Validates a pre-RoPE attention call, uniform (seq_state == nullptr) or ragged, and fills
// its arguments.
int prepare_attn_rope(const kivi_cache* c, int32_t* seq_state, const uint16_t* q, int32_t q_heads, float sm_scale,
                      float rope_base, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                      int32_t num_splits, AttnArgs* pa) {
    if (!std::isfinite(rope_base) || !(rope_base > 0.0f)) return KIVI_ERR_SHAPE;
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if (!(c->flags & KIVI_CODES_4BIT) && c->token_cap > kMaxTokenCapRope2) return KIVI_ERR_UNSUPPORTED;
    if (seq_state == nullptr && (st = check_state(c)) != KIVI_OK) return st;
    if (q_heads <= 0 || q_heads % c->kv_heads != 0) return KIVI_ERR_SHAPE;
    if (num_splits < 0 || num_splits > kMaxSplits) return KIVI_ERR_SHAPE;
    const int32_t splits =
        num_splits > 0 ? num_splits : (seq_state != nullptr ? rope_ragged_splits(c, q_heads) : rope_auto_splits(c, q_heads));
    st = prepare_attn(c, q, q_heads, sm_scale, out, lse, workspace, workspace_bytes, splits, pa, seq_state);
    if (st != KIVI_OK) return st;
    pa->nq = rope_queries_per_block(c, q_heads);
    pa->block_rows = pa->q_rows / pa->nq;
    pa->slot_budget = (int32_t)(pa->nq > 1 ? kTargetBlocksRopeGroup : kTargetBlocksRope);
    pa->rope_base = (double)rope_base;
    return KIVI_OK;
}

int decode_attn_rope(const kivi_cache* c, int32_t* seq_state, const uint16_t* q, int32_t q_heads, float sm_scale,
                     float rope_base, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                     int32_t num_splits, void* stream) {
    AttnArgs a;
    const int st = prepare_attn_rope(c, seq_state, q, q_heads, sm_scale, rope_base, out, lse, workspace,
                                     workspace_bytes, num_splits, &a);
    if (st != KIVI_OK) return st;
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    return hip_status(launch_decode_attn_rope(a, (hipStream_t)stream, t0, t1));
}

int kivi_decode_attn_rope(const kivi_cache* c, const uint16_t* q, int32_t q_heads, float sm_scale,
                          float rope_base, uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                          int32_t num_splits, void* stream) {
    return decode_attn_rope(c, nullptr, q, q_heads, sm_scale, rope_base, out, lse, workspace, workspace_bytes,
                            num_splits, stream);
}

int kivi_decode_attn_rope_ragged(const kivi_cache* c, int32_t* seq_state, const uint16_t* q, int32_t q_heads,
                                 float sm_scale, float rope_base, uint16_t* out, float* lse, void* workspace,
                                 size_t workspace_bytes, int32_t num_splits, void* stream) {
    if (seq_state == nullptr) return KIVI_ERR_NULL;
    return decode_attn_rope(c, seq_state, q, q_heads, sm_scale, rope_base, out, lse, workspace, workspace_bytes,
                            num_splits, stream);
}

int32_t kivi_decode_attn_rope_ragged_splits(const kivi_cache* c, int32_t q_heads) {
    const int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if (q_heads <= 0 || q_heads % c->kv_heads != 0) return KIVI_ERR_SHAPE;
    return rope_ragged_splits(c, q_heads);
}

int32_t kivi_decode_attn_rope_splits(const kivi_cache* c, int32_t q_heads) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_state(c)) != KIVI_OK) return st;
    if (q_heads <= 0 || q_heads % c->kv_heads != 0) return KIVI_ERR_SHAPE;
    return rope_auto_splits(c, q_heads);
}

int32_t kivi_decode_step_splits(const kivi_cache* c, int32_t q_heads, int32_t pre_rope) {
    int st = check_shape(c);
    if (st != KIVI_OK) return st;
    if ((st = check_state(c)) != KIVI_OK) return st;
    if (q_heads <= 0 || q_heads % c->kv_heads != 0) return KIVI_ERR_SHAPE;
    kivi_cache next;
    bool flush;
    if ((st = post_append_state(c, &next, &flush)) != KIVI_OK) return st;
    return pre_rope ? rope_auto_splits(&next, q_heads) : auto_splits(&next, q_heads);
}

size_t kivi_decode_step_workspace(const kivi_cache* c, int32_t q_heads, int32_t num_splits, int32_t pre_rope) {
    if (num_splits < 0) return 0;
    const int32_t s = num_splits > 0 ? num_splits : kivi_decode_step_splits(c, q_heads, pre_rope);
    if (s < 0) return 0;
    kivi_cache next;
    bool flush;
    if (post_append_state(c, &next, &flush) != KIVI_OK) return 0;
    return kivi_decode_attn_workspace(&next, q_heads, s);
}

int kivi_decode_step_rope(kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                          int32_t q_heads, float sm_scale, float rope_base, uint16_t* out, float* lse,
                          void* workspace, size_t workspace_bytes, int32_t num_splits, int32_t* flushed,
                          void* stream) {
    AppendArgs ap;
    kivi_cache next;
    int st = prepare_append(c, k_new, v_new, &ap, &next);
    if (st != KIVI_OK) return st;
    AttnArgs at;   // pre-RoPE attention on the state after the append
    st = prepare_attn_rope(&next, nullptr, q, q_heads, sm_scale, rope_base, out, lse, workspace, workspace_bytes,
                           num_splits, &at);
    if (st != KIVI_OK) return st;
    if (ap.do_flush) {
        if ((st = hip_status(launch_append_flush(ap, (hipStream_t)stream))) != KIVI_OK) return st;
    } else {
        at.k_new = k_new;
        at.v_new = v_new;
        at.k_ring = c->k_res;
        at.v_ring = c->v_res;
        at.new_slot = ap.new_slot;
    }
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    if ((st = hip_status(launch_decode_attn_rope(at, (hipStream_t)stream, t0, t1))) != KIVI_OK) return st;
    commit_state(c, next);
    if (flushed != nullptr) *flushed = ap.do_flush;
    return KIVI_OK;
}

int kivi_decode_step(kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q,
                     int32_t q_heads, float sm_scale, uint16_t* out, float* lse, void* workspace,
                     size_t workspace_bytes, int32_t num_splits, int32_t* flushed, void* stream) {
    AppendArgs ap;
    kivi_cache next;
    int st = prepare_append(c, k_new, v_new, &ap, &next);
    if (st != KIVI_OK) return st;
    AttnArgs at;   // attention on the state after the append
    st = prepare_attn(&next, q, q_heads, sm_scale, out, lse, workspace, workspace_bytes, num_splits, &at);
    if (st != KIVI_OK) return st;
    if (ap.do_flush) {
        if ((st = hip_status(launch_append_flush(ap, (hipStream_t)stream))) != KIVI_OK) return st;
    } else {
        // the new token is residual token next.n_res - 1: attention reads it from k_new /
        // v_new and one workgroup per KV row stores it into its ring slot
        at.k_new = k_new;
        at.v_new = v_new;
        at.k_ring = c->k_res;
        at.v_ring = c->v_res;
        at.new_slot = ap.new_slot;
    }
    hipEvent_t t0, t1;
    take_timing(&t0, &t1);
    if ((st = hip_status(launch_decode_attn(at, (hipStream_t)stream, t0, t1))) != KIVI_OK) return st;
    commit_state(c, next);
    if (flushed != nullptr) *flushed = ap.do_flush;
    return KIVI_OK;
}

}  // extern "C"
