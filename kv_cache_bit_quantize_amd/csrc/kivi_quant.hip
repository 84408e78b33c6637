// kivi_quant.hip -- quantize, prefill, append and group-flush kernels (gfx950).
//
// Keys are quantized per-channel over groups of 32 tokens, values per-token over
// groups of 32 channels (record kv-efficiency/kivi-2bit-llama2-13b-mha-4k, "Quant
// method"; article "Your KV cache doesn't have a bit problem...", paragraphs 2-3).
// The newest R tokens stay in fp16 and whole groups of the oldest residual tokens are
// moved into the quantized history (record, "KV bytes basis").
//
// All kernels use 256-thread workgroups and 16-byte global accesses.
#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

// One key token group held in LDS as fp16 [32][128] -> its 1024-byte code tile + 128 pairs.
// Called by all 256 threads of the workgroup; ends with the codes and pairs stored.
__device__ void quant_k_tile(const uint16_t* __restrict__ tile, float* sh_mn, float* sh_s,
                             uint8_t* __restrict__ codes_dst,      // the group's code tile
                             uint32_t* __restrict__ pairs_dst) {   // 128 (scale, zero) words
    const int tid = threadIdx.x;
    if (tid < kD) {
        float mn = h2f(tile[tid]), mx = mn;
#pragma unroll 8
        for (int t = 1; t < kG; ++t) {
            float v = h2f(tile[t * kD + tid]);
            mn = __builtin_fminf(mn, v);
            mx = __builtin_fmaxf(mx, v);
        }
        GroupQ q = group_params(mn, mx);
        pairs_dst[tid] = q.pair;
        sh_mn[tid] = q.mn;
        sh_s[tid] = q.s;
    }
    __syncthreads();
    // thread -> (token t, 16-channel word w): 32 tokens x 8 words
    const int t = tid >> 3, w = tid & 7;
    const uint4* src = reinterpret_cast<const uint4*>(tile + t * kD + w * 16);
    uint4 a = src[0], b = src[1];
    uint32_t h[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        uint32_t bits = (c & 1) ? (h[c >> 1] >> 16) : (h[c >> 1] & 0xffffu);
        int j = w * 16 + c;
        GroupQ q{sh_mn[j], sh_s[j], 0u};
        word |= code_of(h2f(bits), q) << code_bit(c);
    }
    *reinterpret_cast<uint32_t*>(codes_dst + key_word_offset(t, w)) = word;
}

// Eight consecutive channels of one value token (this thread's share of a 32-channel
// group held by 4 adjacent lanes; lane pairs 2w, 2w+1 hold one 16-channel code word).
// Returns the complete 32-bit code word of the pair (valid in both lanes); *pair gets the
// group's (scale, zero) word (valid in every lane of the 4).  All lanes must call it.
__device__ __forceinline__ uint32_t quant_v_8(uint4 x, int odd, uint32_t* pair) {
    uint32_t h[4] = {x.x, x.y, x.z, x.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = h2f(h[i] & 0xffffu);
        v[2 * i + 1] = h2f(h[i] >> 16);
    }
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = __builtin_fminf(mn, v[i]);
        mx = __builtin_fmaxf(mx, v[i]);
    }
    mn = wave_min_xor(mn, 1, 2);
    mx = wave_max_xor(mx, 1, 2);
    GroupQ q = group_params(mn, mx);
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) bits |= code_of(v[i], q) << code_bit(8 * odd + i);
    *pair = q.pair;
    return bits | (uint32_t)__shfl_xor((int)bits, 1, 64);
}

// ------------------------------------------------------------------ kernels ------

// grid.x = rows * (tokens / 32); one key token group per workgroup.
__global__ __launch_bounds__(kBlock) void quantize_k_kernel(QuantArgs a) {
    __shared__ uint4 tile4[kG * kD / 8];
    __shared__ float sh_mn[kD], sh_s[kD];
    const int groups = a.tokens / kG;
    const int64_t row = blockIdx.x / groups;
    const int g = blockIdx.x % groups;
    const uint16_t* src = a.src + row * a.src_row_stride + (int64_t)g * kG * kD;
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    tile4[threadIdx.x] = s4[threadIdx.x];
    tile4[threadIdx.x + kBlock] = s4[threadIdx.x + kBlock];
    __syncthreads();
    const int dst_tok = a.dst_token_off + g * kG;
    uint8_t* codes = a.k_codes + row * a.token_cap * kRowBytes + (int64_t)(dst_tok / kG) * kTileBytes;
    uint32_t* pairs = reinterpret_cast<uint32_t*>(a.k_sz) + (row * (a.token_cap / kG) + dst_tok / kG) * kD;
    quant_k_tile(reinterpret_cast<const uint16_t*>(tile4), sh_mn, sh_s, codes, pairs);
}

// grid.x = ceil(rows * tokens / 16); 16 value tokens per workgroup, 16 lanes per token.
__global__ __launch_bounds__(kBlock) void quantize_v_kernel(QuantArgs a) {
    const int64_t total = a.rows * (int64_t)a.tokens;
    const int64_t gt = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l16 = threadIdx.x & 15;
    const bool live = gt < total;
    const int64_t row = live ? gt / a.tokens : 0;
    const int t = live ? (int)(gt % a.tokens) : 0;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (live) x = reinterpret_cast<const uint4*>(a.src + row * a.src_row_stride + (int64_t)t * kD)[l16];
    uint32_t pair;
    const uint32_t word = quant_v_8(x, l16 & 1, &pair);
    if (live) {
        const int64_t tok = a.dst_token_off + t;          // token inside the row's history
        if ((l16 & 1) == 0)
            *reinterpret_cast<uint32_t*>(a.v_codes + row * a.token_cap * kRowBytes + value_word_offset(tok, l16 >> 1)) = word;
        if ((l16 & 3) == 0)
            reinterpret_cast<uint32_t*>(a.v_sz)[row * a.token_cap * (kD / kG) + value_pair_index(tok, l16 >> 2)] = pair;
    }
}

// grid.x = ceil(rows * n * 16 / 256): copy tokens [first, first+n) of each row into ring
// slots 0..n-1, keys and values.
__global__ __launch_bounds__(kBlock) void residual_load_kernel(ResidualArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;   // 16-byte chunk index
    const int64_t total = a.rows * (int64_t)a.n * 16;
    if (i >= total) return;
    const int64_t row = i / (a.n * 16);
    const int rem = (int)(i % (a.n * 16));
    const int t = rem >> 4, c = rem & 15;
    const int64_t so = row * a.src_row_stride + (int64_t)(a.first + t) * kD;
    const int64_t d = (row * a.residual_cap + t) * kD;
    reinterpret_cast<uint4*>(a.k_res + d)[c] = reinterpret_cast<const uint4*>(a.k + so)[c];
    reinterpret_cast<uint4*>(a.v_res + d)[c] = reinterpret_cast<const uint4*>(a.v + so)[c];
}

// grid.x = rows.  Optional flush of ring slots [flush_slot, flush_slot+32) into key group
// flush_group / value tokens flush_group*32.., then the new token into new_slot.
__global__ __launch_bounds__(kBlock) void append_flush_kernel(AppendArgs a) {
    __shared__ uint4 tile4[kG * kD / 8];
    __shared__ float sh_mn[kD], sh_s[kD];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    if (a.do_flush) {
        const uint4* kr = reinterpret_cast<const uint4*>(a.k_res + (row * a.residual_cap + a.flush_slot) * kD);
        tile4[tid] = kr[tid];
        tile4[tid + kBlock] = kr[tid + kBlock];
        __syncthreads();
        const int dst_tok = a.flush_group * kG;
        uint8_t* kc = a.k_codes + row * a.token_cap * kRowBytes + (int64_t)a.flush_group * kTileBytes;
        uint32_t* kp = reinterpret_cast<uint32_t*>(a.k_sz) + (row * (a.token_cap / kG) + a.flush_group) * kD;
        quant_k_tile(reinterpret_cast<const uint16_t*>(tile4), sh_mn, sh_s, kc, kp);
        // values: 32 tokens x 16 lanes = two passes of 16 tokens
        const uint4* vr = reinterpret_cast<const uint4*>(a.v_res + (row * a.residual_cap + a.flush_slot) * kD);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int t = pass * 16 + (tid >> 4), l16 = tid & 15;
            uint32_t pair;
            const uint32_t word = quant_v_8(vr[t * 16 + l16], l16 & 1, &pair);
            const int64_t tok = dst_tok + t;
            if ((l16 & 1) == 0)
                *reinterpret_cast<uint32_t*>(a.v_codes + row * a.token_cap * kRowBytes + value_word_offset(tok, l16 >> 1)) = word;
            if ((l16 & 3) == 0)
                reinterpret_cast<uint32_t*>(a.v_sz)[row * a.token_cap * (kD / kG) + value_pair_index(tok, l16 >> 2)] = pair;
        }
        __syncthreads();   // every read of the flushed slots is done before the overwrite
    }
    if (tid < 32) {
        const int c = tid & 15;
        const uint16_t* src = (tid < 16 ? a.k_new : a.v_new) + row * kD;
        uint16_t* dst = (tid < 16 ? a.k_res : a.v_res) + (row * a.residual_cap + a.new_slot) * kD;
        reinterpret_cast<uint4*>(dst)[c] = reinterpret_cast<const uint4*>(src)[c];
    }
}

// ------------------------------------------------------------------ launchers ----

hipError_t launch_quantize_k(const QuantArgs& a, hipStream_t s) {
    const int64_t blocks = a.rows * (int64_t)(a.tokens / kG);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_k_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_quantize_v(const QuantArgs& a, hipStream_t s) {
    const int64_t blocks = (a.rows * (int64_t)a.tokens + 15) / 16;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_v_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_residual_load(const ResidualArgs& a, hipStream_t s) {
    const int64_t blocks = (a.rows * (int64_t)a.n * 16 + kBlock - 1) / kBlock;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(residual_load_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_append_flush(const AppendArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(append_flush_kernel, dim3((unsigned)a.rows), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace kivi
