// Paged decode attention for gfx950.
//
// What it computes: page "面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化",
// section 作品简介 -- each query reads only the valid pages of its own sequence,
// located through that sequence's page mapping and bounded by its true length.
// How the work is split: page "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎",
// section 3 -- a one-pass kernel for short contexts and a partition-plus-reduce
// kernel for long ones.  Both are the same kernel here: a workgroup owns one
// (sequence, KV head, partition); with one partition it writes the output,
// otherwise it writes (m, l, acc) partials and the last workgroup of that
// (sequence, KV head) to finish combines them (log-sum-exp reduce), so a
// decode is always a single launch.
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
//   The V cache keeps the slot innermost (in blocks of 32 slots), so those 8
//   tokens of one value dimension are 16 contiguous bytes: one
//   global_load_dwordx4 per lane per 16 value dimensions, no transposition
//   anywhere, and a chunk's V is one contiguous block.
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

constexpr int kWaves = 8;   // two per SIMD: one wave's compute overlaps the other's load waits
constexpr int kChunk = 32;
constexpr int kDecodeBuffers = 2;   // chunk register sets per wave
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Device-scope (all XCDs) store and load, used only for the split partials.
__device__ __forceinline__ void store_device(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_device(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
__global__ __launch_bounds__(kThreads, 1) void decode_partition_kernel(DecodeArgs a, DecodeItems items) {
    constexpr int KS = D / 32;
    constexpr int NB = D / 16;
    // Workgroups are numbered KV-head fastest: the dispatcher deals
    // consecutive workgroups to the XCDs in turn, so every XCD gets an even
    // share of the work whatever the lengths.  With an item table the grid
    // holds only live (sequence, partition) items, numbered sequence by
    // sequence (an empty workgroup would hold a compute unit that a live one
    // could use); without one it holds every (sequence, partition) pair,
    // partition slowest, so that the empty partitions of short sequences
    // come last.
    const int kvh = blockIdx.x % a.n_kv_heads;
    const int rest = blockIdx.x / a.n_kv_heads;
    int seq, part;
    if (items.n_seqs > 0) {
        int lo = 0, hi = items.n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (items.item0[mid] <= rest) lo = mid;
            else hi = mid - 1;
        }
        seq = lo;
        part = rest - items.item0[lo];
    } else {
        seq = rest % a.n_seqs;
        part = rest / a.n_seqs;
    }
    const int L = a.kv_lens[seq];
    const int t0 = part * a.partition_tokens;
    if (t0 >= L) return;
    const int t1 = min(L, t0 + a.partition_tokens);
    const bool single = (L <= a.partition_tokens) || a.part_m == nullptr;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loop control
    const int m16 = lane & 15;
    const int g = lane >> 4;
    const int Hkv = a.n_kv_heads;
    const int G = a.n_q_heads / Hkv;
    const int P = a.page_size;

    // ---- prologue.  Loads are issued in the order the waits want them: this
    // partition's page ids (kept in a register until the LDS store), Q, and
    // -- when pages hold at least one 32-token chunk, so a chunk never crosses
    // a page -- the wave's first chunk, whose page is read straight from the
    // block table.  Only then the LDS store, the barrier and the Q conversion.
    extern __shared__ int32_t sm_pages[];
    const int sh = a.page_shift;
    const int page_base = t0 >> sh;
    const int32_t* bt = a.block_tables + (int64_t)seq * a.max_pages;
    const int n_pages = ((t1 - 1) >> sh) - page_base + 1;
    const int pt0 = (int)threadIdx.x < n_pages ? bt[page_base + threadIdx.x] : 0;

    // Q as the B operand: lane holds Q[head m16][d = 32s + 8g .. +8], hi/lo.
    const bool hv = m16 < G;
    float4 qraw[2 * KS];
    {
        const float* qrow = a.q + ((int64_t)seq * a.n_q_heads + kvh * G + (hv ? m16 : 0)) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qraw[2 * s] = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * g);
            qraw[2 * s + 1] = *reinterpret_cast<const float4*>(qrow + 32 * s + 8 * g + 4);
        }
    }

    const int64_t page_elems = (int64_t)Hkv * P * D;   // one page of one cache, all heads
    const int VT = v_slot_tile(P);                      // slots per V block
    const uint16_t* kc = a.k_cache;
    const uint16_t* vc = a.v_cache;
    // token row of this lane inside a chunk for K block 0 (block 1 is +4)
    const int tk = 8 * (m16 >> 2) + (m16 & 3);

    // chunk c0's K rows (tokens clamped to L-1) and V^T rows; page_of maps a
    // token to its physical page.  `idle` (uniform) issues the same loads
    // with every lane aimed at the first cell of the pools instead: a few
    // cache-resident lines whose data is never used
    auto load_chunk_with = [&](int c0, ChunkRegs<D>& r, auto page_of, bool idle) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int t = min(c0 + tk + 4 * b, L - 1);
            const uint16_t* row = kc + page_of(t) * page_elems + ((kvh * P + (t & (P - 1))) * D + 8 * g);
            if (idle) row = kc;
#pragma unroll
            for (int s = 0; s < KS; ++s) r.k[b][s] = ld16(row + 32 * s);
        }
        int tv = c0 + 8 * g;
        if (tv > L - 1) tv = (L - 1) & ~7;
        // tokens tv..tv+7 (8-aligned) lie in one V slot block: value dims
        // m16, m16+16, ... are rows T elements apart
        const int vslot = tv & (P - 1);
        const uint16_t* vrow = vc + page_of(tv) * page_elems +
                               (((int64_t)kvh * P + (vslot & ~(VT - 1))) * D + m16 * VT + (vslot & (VT - 1)));
        const int64_t vstep = idle ? 0 : (int64_t)16 * VT;
        if (idle) vrow = vc;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) r.v[nb] = ld16(vrow + nb * vstep);
    };
    auto load_chunk = [&](int c0, ChunkRegs<D>& r, bool idle) __attribute__((always_inline)) {
        load_chunk_with(c0, r, [&](int t) { return sm_pages[(t >> sh) - page_base]; }, idle);
    };

    constexpr int NBUF = kDecodeBuffers;
    constexpr int stride = kWaves * kChunk;
    const int cfirst = t0 + wave * kChunk;
    ChunkRegs<D> r[NBUF];
    const bool chunk_in_page = P >= kChunk;
    if (chunk_in_page && cfirst < t1) {
        const int page0 = bt[cfirst >> sh];
        load_chunk_with(cfirst, r[0], [&](int) { return page0; }, false);
    }
    if ((int)threadIdx.x < n_pages) sm_pages[threadIdx.x] = pt0;
    for (int i = threadIdx.x + blockDim.x; i < n_pages; i += blockDim.x) sm_pages[i] = bt[page_base + i];
    __syncthreads();

    u32x4 qhi[KS], qlo[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const float4 x0 = qraw[2 * s];
        const float4 x1 = qraw[2 * s + 1];
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

    // ---- stream the wave's chunks (wave w takes chunks w, w+kWaves, ...) through
    // kDecodeBuffers register sets, kDecodeBuffers-1 chunks of loads in flight
    // during each compute.  Loads are issued unconditionally (for a chunk past
    // the wave's last one they are idle loads of one cache-resident line), so
    // every path issues the same loads and the in-order vmcnt accounting lets a
    // chunk's compute wait for its own loads only.
    if (cfirst < t1) {
        const int last_c = cfirst + ((t1 - 1 - cfirst) / stride) * stride;
        auto load_next = [&](int c, ChunkRegs<D>& r) __attribute__((always_inline)) {
            load_chunk(min(c, last_c), r, c > last_c);
        };
        if (!chunk_in_page) load_chunk(cfirst, r[0], false);
#pragma unroll
        for (int j = 1; j < NBUF - 1; ++j) load_next(cfirst + j * stride, r[j]);
        for (int it = 0;; it += NBUF) {
            bool done = false;
#pragma unroll
            for (int j = 0; j < NBUF; ++j) {
                const int cj = cfirst + (it + j) * stride;
                if (cj >= t1) {
                    done = true;
                    break;
                }
                load_next(cj + (NBUF - 1) * stride, r[(j + NBUF - 1) % NBUF]);
                compute_chunk(cj, r[j]);
            }
            if (done) break;
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
            store_device(a.part_acc + pi * D + d, num);
            if (d == 0) {
                store_device(a.part_m + pi, M);
                store_device(a.part_l + pi, den);
            }
        }
    }
    if (single) return;

    // ---- fused log-sum-exp reduce.  The partials above are device-scope
    // stores (written through to the device coherence point, past the
    // per-XCD L2s); each wave waits until its stores are acknowledged, the
    // barrier makes that true for the whole workgroup, and only then is the
    // (device-scope) completion counter of this (sequence, KV head) bumped.
    // The workgroup that brings the counter to the partition count reads all
    // partials with device-scope loads, writes the output and puts the counter
    // back to zero for the next call.  No L2 write-back or invalidate is needed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int s_last;
    const int np = (L + a.partition_tokens - 1) / a.partition_tokens;
    int32_t* counter = a.counters + seq * Hkv + kvh;
    if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1) == np - 1);
    __syncthreads();
    if (!s_last) return;
    constexpr int kFast = 16;   // partitions combined with one round of loads
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int h = idx / D;
        const int d = idx - h * D;
        const int qh = kvh * G + h;
        const int64_t base = ((int64_t)seq * a.n_q_heads + qh) * a.n_part;
        float num = 0.0f, den = 0.0f;
        if (np <= kFast) {
            float pm[kFast], pl[kFast], px[kFast];
#pragma unroll
            for (int p = 0; p < kFast; ++p) {
                if (p < np) {
                    pm[p] = load_device(a.part_m + base + p);
                    pl[p] = load_device(a.part_l + base + p);
                    px[p] = load_device(a.part_acc + (base + p) * D + d);
                }
            }
            float M = pm[0];
#pragma unroll
            for (int p = 1; p < kFast; ++p)
                if (p < np) M = fmaxf(M, pm[p]);
#pragma unroll
            for (int p = 0; p < kFast; ++p) {
                if (p < np) {
                    const float f = __builtin_amdgcn_exp2f(pm[p] - M);
                    num += f * px[p];
                    den += f * pl[p];
                }
            }
        } else {
            // the maximum first, then the fold in ascending partition order,
            // kFast partitions' loads in flight per round trip
            float M = -INFINITY;
            for (int p0 = 0; p0 < np; p0 += kFast) {
                float pm[kFast];
#pragma unroll
                for (int p = 0; p < kFast; ++p) pm[p] = load_device(a.part_m + base + min(p0 + p, np - 1));
#pragma unroll
                for (int p = 0; p < kFast; ++p) M = fmaxf(M, pm[p]);
            }
            for (int p0 = 0; p0 < np; p0 += kFast) {
                float pm[kFast], pl[kFast], px[kFast];
#pragma unroll
                for (int p = 0; p < kFast; ++p) {
                    const int q = min(p0 + p, np - 1);
                    pm[p] = load_device(a.part_m + base + q);
                    pl[p] = load_device(a.part_l + base + q);
                    px[p] = load_device(a.part_acc + (base + q) * D + d);
                }
#pragma unroll
                for (int p = 0; p < kFast; ++p) {
                    if (p0 + p < np) {
                        const float f = __builtin_amdgcn_exp2f(pm[p] - M);
                        num += f * px[p];
                        den += f * pl[p];
                    }
                }
            }
        }
        a.out[((int64_t)seq * a.n_q_heads + qh) * D + d] = num / den;
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int decode_page_table_entries(int partition_tokens, int page_size) {
    // a partition starting at a multiple of partition_tokens touches at most
    // ceil(partition_tokens / P) + 1 pages
    return (partition_tokens + page_size - 1) / page_size + 1;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodeItems& items, int64_t n_workgroups,
                         hipStream_t stream) {
    const dim3 grid((unsigned)n_workgroups);
    const size_t lds = sizeof(int32_t) * (size_t)decode_page_table_entries(a.partition_tokens, a.page_size);
    if (a.head_dim == 128)
        hipLaunchKernelGGL(decode_partition_kernel<128>, grid, dim3(kThreads), lds, stream, a, items);
    else
        hipLaunchKernelGGL(decode_partition_kernel<64>, grid, dim3(kThreads), lds, stream, a, items);
    return hipGetLastError();
}


}  // namespace pa
