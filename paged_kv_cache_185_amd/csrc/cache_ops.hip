// Reshape-and-cache and block copy ("CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎",
// section 3: fused kernels that write new tokens' K/V into their blocks and
// copy blocks for copy-on-write sharing, section 2).
//
// Both kernels move bits; the only arithmetic is the float32 -> binary16
// conversion (v_cvt_f16_f32, round to nearest even) for float32 sources.
#include "pa_internal.h"

namespace pa {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (16 tokens, KV head).  K rows are contiguous in the cache:
// each 16-byte chunk of a token's row is one store.  V is stored with the slot
// innermost, so V goes through LDS as [d][token] and each run of 8 tokens whose
// slots are consecutive and 8-aligned (the usual case: a sequence's new tokens
// fill its pages in order) becomes one 16-byte store per d row; any other slot
// pattern falls back to 2-byte stores.
constexpr int kRcTokens = 16;
constexpr int kRcThreads = 256;

template <bool kSrcF32, int D>
__global__ __launch_bounds__(kRcThreads) void reshape_and_cache_kernel(
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache, const void* __restrict__ k_new,
    const void* __restrict__ v_new, const int32_t* __restrict__ slots, int32_t n_tokens,
    int32_t n_kv_heads, int32_t page_shift) {
    constexpr int CH = D / 8;
    constexpr int kRow = kRcTokens + 8;   // LDS row of one d: 48 bytes, 16-byte aligned
    __shared__ __align__(16) uint16_t sv[D * kRow];
    __shared__ int32_t sslot[kRcTokens];
    const int h = blockIdx.y;
    const int tok0 = blockIdx.x * kRcTokens;
    const int tid = threadIdx.x;
    const int P = 1 << page_shift;
    if (tid < kRcTokens) sslot[tid] = tok0 + tid < n_tokens ? slots[tok0 + tid] : -1;
    __syncthreads();

    for (int task = tid; task < kRcTokens * CH; task += kRcThreads) {
        const int tl = task / CH;
        const int c = task - tl * CH;
        const int32_t slot = sslot[tl];
        if (slot < 0) continue;
        const int64_t src = ((int64_t)(tok0 + tl) * n_kv_heads + h) * D + 8 * c;
        uint16_t kv[8], vv[8];
        if constexpr (kSrcF32) {
            const float* ks = reinterpret_cast<const float*>(k_new) + src;
            const float* vs = reinterpret_cast<const float*>(v_new) + src;
            const float4 k0 = *reinterpret_cast<const float4*>(ks);
            const float4 k1 = *reinterpret_cast<const float4*>(ks + 4);
            const float4 v0 = *reinterpret_cast<const float4*>(vs);
            const float4 v1 = *reinterpret_cast<const float4*>(vs + 4);
            const float kf[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
            const float vf[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kv[e] = __builtin_bit_cast(uint16_t, (_Float16)kf[e]);
                vv[e] = __builtin_bit_cast(uint16_t, (_Float16)vf[e]);
            }
        } else {
            const u32x4 kk = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(k_new) + src);
            const u32x4 vw = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(v_new) + src);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                kv[2 * w] = (uint16_t)(kk[w] & 0xffffu);
                kv[2 * w + 1] = (uint16_t)(kk[w] >> 16);
                vv[2 * w] = (uint16_t)(vw[w] & 0xffffu);
                vv[2 * w + 1] = (uint16_t)(vw[w] >> 16);
            }
        }
        u32x4 kout;
#pragma unroll
        for (int w = 0; w < 4; ++w) kout[w] = (uint32_t)kv[2 * w] | ((uint32_t)kv[2 * w + 1] << 16);
        const int64_t page = slot >> page_shift;
        const int off = slot & (P - 1);
        *reinterpret_cast<u32x4*>(k_cache + ((page * n_kv_heads + h) * P + off) * D + 8 * c) = kout;
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[(8 * c + e) * kRow + tl] = vv[e];
    }
    __syncthreads();

    // V rows: task (d, g) covers tokens 8g..8g+7 of row d; lanes of a wave
    // take consecutive g, so a run of slots in order is written contiguously
    constexpr int NG = kRcTokens / 8;
    for (int task = tid; task < D * NG; task += kRcThreads) {
        const int d = task / NG;
        const int g = task % NG;
        const int32_t s0 = sslot[8 * g];
        bool run = s0 >= 0 && (s0 & 7) == 0;
#pragma unroll
        for (int j = 1; j < 8; ++j) run = run && sslot[8 * g + j] == s0 + j;
        if (run) {
            const int64_t page = s0 >> page_shift;
            const int off = s0 & (P - 1);
            // 8 consecutive slots from an 8-aligned one lie in one slot block
            *reinterpret_cast<u32x4*>(v_cache + v_elem_offset(page, h, d, off, n_kv_heads, P, D)) =
                *reinterpret_cast<const u32x4*>(&sv[d * kRow + 8 * g]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int32_t sj = sslot[8 * g + j];
                if (sj < 0) continue;
                const int64_t page = sj >> page_shift;
                v_cache[v_elem_offset(page, h, d, sj & (P - 1), n_kv_heads, P, D)] = sv[d * kRow + 8 * g + j];
            }
        }
    }
}

// Page copies between two page arrays of the same layout (src and dst base per
// layer for K and V): the same array for copy-on-write, the device pool and a
// pinned host reserve for swap.
struct CopyPagesArgs {
    const uint16_t* src_k[kMaxCopyLayers];
    uint16_t* dst_k[kMaxCopyLayers];
    const uint16_t* src_v[kMaxCopyLayers];
    uint16_t* dst_v[kMaxCopyLayers];
    int32_t pairs[2 * kMaxCopyPairs];
};

constexpr int kCopyBytesPerBlock = 16384;

// grid: (ceil(page_bytes / 16 KiB), n_pairs, 2 * n_layers); 16-byte vector copies.
__global__ __launch_bounds__(256) void copy_pages_kernel(CopyPagesArgs args, int64_t page_bytes) {
    const int pair = blockIdx.y;
    const int layer = blockIdx.z >> 1;
    const bool is_v = blockIdx.z & 1;
    const char* src = reinterpret_cast<const char*>(is_v ? args.src_v[layer] : args.src_k[layer]) +
                      (int64_t)args.pairs[2 * pair] * page_bytes;
    char* dst = reinterpret_cast<char*>(is_v ? args.dst_v[layer] : args.dst_k[layer]) +
                (int64_t)args.pairs[2 * pair + 1] * page_bytes;
    const int64_t begin = (int64_t)blockIdx.x * kCopyBytesPerBlock;
    const int64_t end = begin + kCopyBytesPerBlock < page_bytes ? begin + kCopyBytesPerBlock : page_bytes;
    for (int64_t off = begin + (int64_t)threadIdx.x * 16; off < end; off += 256 * 16)
        *reinterpret_cast<u32x4*>(dst + off) = *reinterpret_cast<const u32x4*>(src + off);
}

__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ out,
                                                        const int32_t* __restrict__ token_row,
                                                        int32_t n_tokens, int32_t row_elems) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tok = i / row_elems;
    if (tok >= n_tokens) return;
    if (token_row[tok] < 0) out[i] = 0.0f;
}

}  // namespace

hipError_t launch_reshape_and_cache(void* k_cache, void* v_cache, const void* k_new,
                                    const void* v_new, bool src_f32, const int32_t* slots,
                                    int32_t n_tokens, int32_t n_kv_heads, int32_t page_size,
                                    int32_t head_dim, hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    const dim3 grid((unsigned)((n_tokens + kRcTokens - 1) / kRcTokens), (unsigned)n_kv_heads);
    auto* kc = (uint16_t*)k_cache;
    auto* vc = (uint16_t*)v_cache;
    if (head_dim == 128) {
        if (src_f32)
            hipLaunchKernelGGL((reshape_and_cache_kernel<true, 128>), grid, dim3(kRcThreads), 0, stream, kc, vc,
                               k_new, v_new, slots, n_tokens, n_kv_heads, shift);
        else
            hipLaunchKernelGGL((reshape_and_cache_kernel<false, 128>), grid, dim3(kRcThreads), 0, stream, kc, vc,
                               k_new, v_new, slots, n_tokens, n_kv_heads, shift);
    } else {
        if (src_f32)
            hipLaunchKernelGGL((reshape_and_cache_kernel<true, 64>), grid, dim3(kRcThreads), 0, stream, kc, vc,
                               k_new, v_new, slots, n_tokens, n_kv_heads, shift);
        else
            hipLaunchKernelGGL((reshape_and_cache_kernel<false, 64>), grid, dim3(kRcThreads), 0, stream, kc, vc,
                               k_new, v_new, slots, n_tokens, n_kv_heads, shift);
    }
    return hipGetLastError();
}

hipError_t launch_copy_pages(void* const* src_k, void* const* dst_k, void* const* src_v,
                             void* const* dst_v, int32_t n_layers, const int32_t* pairs, int32_t n_pairs,
                             int64_t page_bytes, hipStream_t stream) {
    for (int32_t l0 = 0; l0 < n_layers; l0 += kMaxCopyLayers) {
        const int32_t nl = n_layers - l0 < kMaxCopyLayers ? n_layers - l0 : kMaxCopyLayers;
        for (int32_t p0 = 0; p0 < n_pairs; p0 += kMaxCopyPairs) {
            const int32_t np = n_pairs - p0 < kMaxCopyPairs ? n_pairs - p0 : kMaxCopyPairs;
            CopyPagesArgs args{};
            for (int32_t l = 0; l < nl; ++l) {
                args.src_k[l] = (const uint16_t*)src_k[l0 + l];
                args.dst_k[l] = (uint16_t*)dst_k[l0 + l];
                args.src_v[l] = (const uint16_t*)src_v[l0 + l];
                args.dst_v[l] = (uint16_t*)dst_v[l0 + l];
            }
            for (int32_t i = 0; i < 2 * np; ++i) args.pairs[i] = pairs[2 * p0 + i];
            const dim3 grid((unsigned)((page_bytes + kCopyBytesPerBlock - 1) / kCopyBytesPerBlock),
                            (unsigned)np, (unsigned)(2 * nl));
            hipLaunchKernelGGL(copy_pages_kernel, grid, dim3(256), 0, stream, args, page_bytes);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t n_layers,
                              const int32_t* pairs, int32_t n_pairs, int64_t page_bytes,
                              hipStream_t stream) {
    return launch_copy_pages(k_caches, k_caches, v_caches, v_caches, n_layers, pairs, n_pairs,
                             page_bytes, stream);
}

hipError_t launch_zero_rows(float* out, const int32_t* token_row, int32_t n_tokens,
                            int32_t row_elems, hipStream_t stream) {
    const int64_t n = (int64_t)n_tokens * row_elems;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       out, token_row, n_tokens, row_elems);
    return hipGetLastError();
}

}  // namespace pa
