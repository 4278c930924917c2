// Paged decode attention for gfx950.
//
// What it computes: page "面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化",
// section 作品简介 -- each query reads only the valid pages of its own sequence,
// located through that sequence's page mapping and bounded by its true length.
// How the work is split: page "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎",
// section 3 -- a one-pass kernel for short contexts and a partition-plus-reduce
// kernel for long ones.  Both are the same kernel here: a workgroup owns one
// (sequence, KV head, partition); with one partition it writes the output,
// otherwise (m, l, acc) partials that decode_reduce_kernel combines.
//
// Design (MI355X):
// * All G = Hq/Hkv query heads of a KV head are served by one pass over each
//   KV cell, so valid K/V bytes are read from HBM once.
// * Scores and P.V run on MFMA v_mfma_f32_16x16x32_f16.  The score block is
//   computed transposed, S^T = K Q^T (rows = 16 tokens, columns = heads), so a
//   lane's C registers belong to one head: the softmax state (m, l) and the
//   output accumulator O^T = V^T P^T are per-lane scalars, and P^T leaves the
//   score registers already in the B-operand layout of the P.V product.
// * Token-to-row assignment inside a 32-token chunk is chosen so that lane
//   group g (lanes 16g..16g+15) ends up holding tokens 8g..8g+7 of the chunk.
//   The V cache keeps the slot innermost, so those 8 tokens of one value
//   dimension are 16 contiguous bytes: one global_load_dwordx4 per lane per
//   16 value dimensions, no transposition anywhere.
// * Q (fp32) enters the score MFMA as a binary16 hi/lo pair (q = hi + lo), two
//   MFMAs per block, so Q is carried to ~22 bits; P is rounded to binary16 for
//   the P.V product and the row sum uses the same rounded values.
// * Softmax runs in the log2 domain (scale * log2 e folded into the scores).
// * Invalid cells (beyond the true length, including NaN padding inside the
//   last page) are removed by select: scores become -inf and the matching V
//   halves are zeroed, so no NaN can reach an MFMA.  Loads for tokens past
//   the true length are redirected to the last valid token's page.
#include <math.h>

#include "pa_internal.h"

namespace pa {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kChunk = 32;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

template <int D>
struct ChunkRegs {
    u32x4 k[2][D / 32];   // K rows, two 16-token blocks, D/32 k-steps
    u32x4 v[D / 16];      // V^T rows, D/16 blocks of 16 value dims
};

template <int D>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeArgs a) {
    constexpr int KS = D / 32;
    constexpr int NB = D / 16;
    const int part = blockIdx.x;
    const int kvh = blockIdx.y;
    const int seq = blockIdx.z;
    const int L = a.kv_lens[seq];
    const int t0 = part * a.partition_tokens;
    if (t0 >= L) return;
    const int t1 = min(L, t0 + a.partition_tokens);
    const bool single = (L <= a.partition_tokens) || a.part_m == nullptr;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m16 = lane & 15;
    const int g = lane >> 4;
    const int Hkv = a.n_kv_heads;
    const int G = a.n_q_heads / Hkv;
    const int P = a.page_size;

    // ---- Q as the B operand: lane holds Q[head m16][d = 32s + 8g .. +8], hi/lo.
    u32x4 qhi[KS], qlo[KS];
    {
        const bool hv = m16 < G;
        const float* qrow = a.q + ((int64_t)seq * a.n_q_heads + kvh * G + (hv ? m16 : 0)) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * g);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * g + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            f16x8 h, l;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = hv ? xs[e] : 0.0f;
                const _Float16 hi = (_Float16)x;
                h[e] = hi;
                l[e] = (_Float16)(x - (float)hi);
            }
            qhi[s] = __builtin_bit_cast(u32x4, h);
            qlo[s] = __builtin_bit_cast(u32x4, l);
        }
    }

    const int32_t* bt = a.block_tables + (int64_t)seq * a.max_pages;
    const uint16_t* kc = a.k_cache;
    const uint16_t* vc = a.v_cache;
    // token row of this lane inside a chunk for K block 0 (block 1 is +4)
    const int tk = 8 * (m16 >> 2) + (m16 & 3);

    auto load_chunk = [&](int c0, ChunkRegs<D>& r) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int t = min(c0 + tk + 4 * b, L - 1);
            const int page = bt[t / P];
            const uint16_t* row = kc + (((int64_t)page * Hkv + kvh) * P + (t % P)) * D + 8 * g;
#pragma unroll
            for (int s = 0; s < KS; ++s) r.k[b][s] = ld16(row + 32 * s);
        }
        int tv = c0 + 8 * g;
        if (tv > L - 1) tv = (L - 1) & ~7;
        const int vpage = bt[tv / P];
        const uint16_t* vrow = vc + (((int64_t)vpage * Hkv + kvh) * D + m16) * P + (tv % P);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) r.v[nb] = ld16(vrow + (int64_t)16 * nb * P);
    };

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_chunk = [&](int c0, ChunkRegs<D>& r) {
        f32x4 sc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                c = mfma16(r.k[b][s], qhi[s], c);
                c = mfma16(r.k[b][s], qlo[s], c);
            }
            sc[b] = c;
        }
        const int tb = c0 + 8 * g;   // first token held by this lane group
        float sv[8];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = sc[b][i] * a.scale_log2;
                sv[4 * b + i] = (tb + 4 * b + i < L) ? x : -INFINITY;
            }
        float mx = sv[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        f16x8 pb;
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const _Float16 p = (_Float16)__builtin_amdgcn_exp2f(sv[e] - m_new);
            pb[e] = p;
            psum += (float)p;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (c0 + kChunk > L) {
            // zero V halves of tokens >= L so NaN padding never meets a zero weight
            const int nvalid = max(0, min(8, L - tb));
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t mk = (2 * w < nvalid ? 0x0000ffffu : 0u) |
                                    (2 * w + 1 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) r.v[nb][w] &= mk;
            }
        }
        const u32x4 pbits = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            acc[nb] *= alpha;
            acc[nb] = mfma16(r.v[nb], pbits, acc[nb]);
        }
    };

    // ---- stream the wave's chunks (wave w takes chunks w, w+4, ...), two
    // register sets so the next chunk's loads are in flight during compute.
    const int stride = kWaves * kChunk;
    int c = t0 + wave * kChunk;
    if (c < t1) {
        ChunkRegs<D> ra, rb;
        load_chunk(c, ra);
        while (true) {
            const int cb = c + stride;
            if (cb < t1) load_chunk(cb, rb);
            compute_chunk(c, ra);
            if (cb >= t1) break;
            const int ca = cb + stride;
            if (ca < t1) load_chunk(ca, ra);
            compute_chunk(cb, rb);
            if (ca >= t1) break;
            c = ca;
        }
    }

    // row sums over the four lane groups (m_run is already uniform across them)
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // ---- combine the waves of the workgroup
    __shared__ float sm_m[kWaves][16];
    __shared__ float sm_l[kWaves][16];
    __shared__ float sm_acc[kWaves][D][17];
    if (g == 0) {
        sm_m[wave][m16] = m_run;
        sm_l[wave][m16] = l_run;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_acc[wave][16 * nb + 4 * g + i][m16] = acc[nb][i];
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        float M = sm_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm_m[w][h];
            const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            num += f * sm_acc[w][d][h];
            den += f * sm_l[w][h];
        }
        const int qh = kvh * G + h;
        if (single) {
            a.out[((int64_t)seq * a.n_q_heads + qh) * D + d] = num / den;
        } else {
            const int64_t pi = ((int64_t)seq * a.n_q_heads + qh) * a.n_part + part;
            a.part_acc[pi * D + d] = num;
            if (d == 0) {
                a.part_m[pi] = M;
                a.part_l[pi] = den;
            }
        }
    }
}

// One workgroup of D threads per (sequence, query head): log-sum-exp combine
// of the sequence's partitions.  Sequences with a single partition were
// written by the partition kernel and are skipped.
template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
    const int seq = blockIdx.x;
    const int qh = blockIdx.y;
    const int d = threadIdx.x;
    const int L = a.kv_lens[seq];
    const int np = (L + a.partition_tokens - 1) / a.partition_tokens;
    if (np <= 1) return;
    const int64_t base = ((int64_t)seq * a.n_q_heads + qh) * a.n_part;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p) M = fmaxf(M, a.part_m[base + p]);
    float num = 0.0f, den = 0.0f;
    for (int p = 0; p < np; ++p) {
        const float f = __builtin_amdgcn_exp2f(a.part_m[base + p] - M);
        num += f * a.part_acc[(base + p) * D + d];
        den += f * a.part_l[base + p];
    }
    a.out[((int64_t)seq * a.n_q_heads + qh) * D + d] = num / den;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_part, (unsigned)a.n_kv_heads, (unsigned)a.n_seqs);
    if (a.head_dim == 128)
        hipLaunchKernelGGL(decode_partition_kernel<128>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(decode_partition_kernel<64>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_seqs, (unsigned)a.n_q_heads);
    if (a.head_dim == 128)
        hipLaunchKernelGGL(decode_reduce_kernel<128>, grid, dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL(decode_reduce_kernel<64>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
