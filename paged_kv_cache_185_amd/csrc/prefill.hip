// UA paged prefill attention for gfx950.
//
// What it computes: page "面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化",
// section 作品简介 -- every token of a mixed ubatch carries its own sequence's
// page mapping (block-table row) and true KV length, and attends only to the
// valid cells of that sequence: cells t < min(kv_len, pos + 1).
//
// Design (MI355X):
// * The host groups each sequence's tokens into tiles of 256 query rows
//   (256/G tokens x G heads of one KV head).  A workgroup (8 waves) owns one
//   (tile, KV split, KV head); wave w owns 32 query columns.  The tile's
//   tokens are found on the device by a ballot scan of token_row over the
//   tile's ubatch index range, so no plan has to be copied to the device.
//   Workgroups are numbered KV-head-fastest: on an 8-XCD part with 8 KV heads
//   every workgroup of one head lands on the same XCD, and the tiles and
//   splits of that head share its K/V through that XCD's L2.
// * K and V tiles of 64 keys are staged through LDS (double buffered, XOR
//   swizzled in 16-byte units) and shared by the 8 waves.  Global loads run
//   two tiles ahead of the MFMA work (two register sets), so about two
//   tiles' worth of compute covers each load's latency.
// * Both products run on v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//   Scores are computed transposed, S^T = K Q^T (rows = keys, columns =
//   queries): each lane's C registers belong to one query column, so the
//   row max / row sum need one cross-half exchange, and P^T is already in the
//   B-operand layout of O^T = V^T P^T.  The key order of the score rows is
//   permuted (bits 2 and 3 of the row index swapped) so that the 8 keys a lane
//   holds for each P.V k-step are contiguous, which lets the V operand be one
//   16-byte LDS read from the slot-innermost V tile.
// * Q is multiplied by scale*log2(e) and rounded to binary16 once, so scores
//   come out of the MFMA already in the log2 domain; P is rounded to binary16
//   for the P.V product; row sums and accumulators are fp32.
// * The running maximum is raised only when a new score exceeds it by more
//   than 8 (log2 units): until then P <= 2^8 stays exact enough in binary16
//   and the output rescale (a multiply per accumulator) is skipped.
// * Masking is by select (scores -> -inf), and only on tiles that cross some
//   token's visible end.  V cells at or past the tile's visible end are zeroed
//   in registers before they reach LDS, so NaN padding never meets a zero
//   weight.
// * Long KV ranges are split across workgroups; each split writes (m, l, acc)
//   partials that prefill_reduce_kernel combines by log-sum-exp.
#include <math.h>

#include "pa_internal.h"

namespace pa {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;          // query rows (token x head) per tile
constexpr int kKvTile = kPrefillKvTile;     // 64 keys per iteration
constexpr float kRescaleSlack = 8.0f;       // log2 units the max may lag by

struct TileList {
    PrefillTile t[kMaxTilesPerLaunch];
};

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// score row i of a 32-key block <-> key offset (bits 2 and 3 swapped)
__device__ __forceinline__ int kappa(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

template <int D>
struct Smem {
    u32x4 k[2][kKvTile * D / 8];   // [buf][key][D/8 chunks], chunk swizzled by key % 8
    u32x4 v[2][D * kKvTile / 8];   // [buf][d][8 chunks of 8 keys], chunk swizzled by d % 8
    int32_t tok[kRows];
    int32_t min_vis;
};

template <int D>
struct Staging {
    static constexpr int KC = kKvTile * D / 8 / kThreads;   // 16-byte chunks per thread (K)
    static constexpr int VC = D * kKvTile / 8 / kThreads;   // (V)
    u32x4 k[KC];
    u32x4 v[VC];
};

template <int D, int G>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a, TileList tl) {
    constexpr int TPW = 32 / G;       // tokens per wave
    constexpr int KS = D / 16;        // k-steps of the score product
    constexpr int DB = D / 32;        // 32-row output blocks
    constexpr int CPR = D / 8;        // 16-byte chunks per K row

    const int Hkv = a.n_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int rest = blockIdx.x / Hkv;
    const int tile_idx = rest % a.n_tiles;
    const int split = rest / a.n_tiles;
    const PrefillTile tile = tl.t[tile_idx];
    if (split >= tile.n_splits) return;
    const int kv_begin = split * a.split_tokens;
    const int kv_end = min(tile.kv_end, kv_begin + a.split_tokens);

    __shared__ Smem<D> sm;
    extern __shared__ int32_t sm_pages[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int hh = lane >> 5;
    const int P = a.page_size;

    // ---- tokens of this tile (ballot scan of token_row[first..last]) and the
    // page ids of this split's key range
    if (wave == 0) {
        int found = 0;
        for (int base = tile.first; base <= tile.last && found < tile.count; base += 64) {
            const int i = base + lane;
            const bool hit = (i <= tile.last) && a.token_row[i] == tile.row;
            const uint64_t mask = __ballot(hit);
            const int before = __popcll(mask & ((1ull << lane) - 1ull));
            if (hit && found + before < tile.count) sm.tok[found + before] = i;
            found += __popcll(mask);
        }
    }
    if (tid == 0) sm.min_vis = kv_end;
    const int page_base = kv_begin / P;
    {
        const int32_t* bt = a.block_tables + (int64_t)tile.row * a.max_pages;
        const int n_pages = (kv_end - 1) / P - page_base + 1;
        for (int i = tid; i < n_pages; i += kThreads) sm_pages[i] = bt[page_base + i];
    }
    __syncthreads();

    // ---- this lane's query column
    const int ti = wave * TPW + col / G;
    const int hq = col % G;
    const int tok = ti < tile.count ? sm.tok[ti] : -1;
    int n_vis = 0;
    if (tok >= 0) n_vis = min(a.token_kv_len[tok], a.token_pos[tok] + 1);
    const int qh = kvh * G + hq;
    if (tok >= 0) atomicMin(&sm.min_vis, n_vis);

    u32x4 qb[KS];
    {
        const float* qrow = a.q + ((int64_t)(tok >= 0 ? tok : 0) * a.n_q_heads + qh) * D;
        const float qs = tok >= 0 ? a.scale_log2 : 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * hh;
            const float4 x0 = *reinterpret_cast<const float4*>(qrow + d0);
            const float4 x1 = *reinterpret_cast<const float4*>(qrow + d0 + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            f16x8 h;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (_Float16)(xs[e] * qs);
            qb[ks] = __builtin_bit_cast(u32x4, h);
        }
    }

    const uint16_t* kc = a.k_cache;
    const uint16_t* vc = a.v_cache;

    // ---- global -> registers for one KV tile starting at key t0
    auto load_tile = [&](int t0, Staging<D>& st) {
#pragma unroll
        for (int i = 0; i < Staging<D>::KC; ++i) {
            const int id = tid + kThreads * i;
            const int key = id / CPR;
            const int c = id - key * CPR;
            const int t = min(t0 + key, kv_end - 1);
            const int page = sm_pages[t / P - page_base];
            st.k[i] = *reinterpret_cast<const u32x4*>(
                kc + (((int64_t)page * Hkv + kvh) * P + (t % P)) * D + 8 * c);
        }
#pragma unroll
        for (int i = 0; i < Staging<D>::VC; ++i) {
            const int id = tid + kThreads * i;
            const int d = id >> 3;
            const int c = id & 7;
            const int tb = t0 + 8 * c;
            const int tv = tb < kv_end ? tb : ((kv_end - 1) & ~7);
            const int page = sm_pages[tv / P - page_base];
            u32x4 x = *reinterpret_cast<const u32x4*>(
                vc + (((int64_t)page * Hkv + kvh) * D + d) * P + (tv % P));
            const int nvalid = max(0, min(8, kv_end - tb));
            if (nvalid < 8) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t mk = (2 * w < nvalid ? 0x0000ffffu : 0u) |
                                        (2 * w + 1 < nvalid ? 0xffff0000u : 0u);
                    x[w] &= mk;
                }
            }
            st.v[i] = x;
        }
    };
    auto store_tile = [&](int buf, const Staging<D>& st) {
#pragma unroll
        for (int i = 0; i < Staging<D>::KC; ++i) {
            const int id = tid + kThreads * i;
            const int key = id / CPR;
            const int c = id - key * CPR;
            sm.k[buf][key * CPR + (c ^ (key & 7))] = st.k[i];
        }
#pragma unroll
        for (int i = 0; i < Staging<D>::VC; ++i) {
            const int id = tid + kThreads * i;
            const int d = id >> 3;
            const int c = id & 7;
            sm.v[buf][d * 8 + (c ^ (d & 7))] = st.v[i];
        }
    };

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;

    // one 64-key tile from LDS buffer `buf`, keys t0..t0+63
    auto compute_tile = [&](int buf, int t0, bool full) {
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
            const int krow = 32 * kb + kappa(col);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = 2 * ks + hh;
                const u32x4 kop = sm.k[buf][krow * CPR + (c ^ (krow & 7))];
                s[kb] = mfma32(kop, qb[ks], s[kb]);
            }
        }
        if (!full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = t0 + 32 * kb + 16 * (r >> 3) + 8 * hh + (r & 7);
                    s[kb][r] = key < n_vis ? s[kb][r] : -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // raise the running max only when the new one is well above it
        const bool raise = mx > m_run + kRescaleSlack;
        if (__ballot(raise)) {
            const float m_new = raise ? mx : m_run;
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= alpha;
            m_run = m_new;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        u32x4 pb[4];
        float psum = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            f16x8 p;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(s[ks >> 1][8 * (ks & 1) + e] - m_use);
                psum += pe;
                p[e] = (_Float16)pe;
            }
            pb[ks] = __builtin_bit_cast(u32x4, p);
        }
        l_run += psum;
        // O^T += V^T P^T
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = 2 * ks + hh;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = 32 * db + col;
                const u32x4 vop = sm.v[buf][d * 8 + (c ^ (d & 7))];
                acc[db] = mfma32(vop, pb[ks], acc[db]);
            }
        }
    };

    __syncthreads();   // sm.min_vis complete
    const int min_vis = min(sm.min_vis, kv_end);
    const int n_tiles = (kv_end - kv_begin + kKvTile - 1) / kKvTile;

    // ---- pipeline: registers hold tiles it+1 and it+2 while tile it is
    // computed from LDS; one barrier per tile
    Staging<D> sa, sb;
    load_tile(kv_begin, sa);
    if (n_tiles > 1) load_tile(kv_begin + kKvTile, sb);
    store_tile(0, sa);
    __syncthreads();
    for (int it = 0; it < n_tiles; it += 2) {
        {   // even tile: computed from buffer 0; sb holds tile it+1
            const int t0 = kv_begin + it * kKvTile;
            if (it + 2 < n_tiles) load_tile(t0 + 2 * kKvTile, sa);
            compute_tile(0, t0, t0 + kKvTile <= min_vis);
            if (it + 1 < n_tiles) store_tile(1, sb);
            __syncthreads();
        }
        if (it + 1 < n_tiles) {   // odd tile: computed from buffer 1; sa holds tile it+2
            const int t0 = kv_begin + (it + 1) * kKvTile;
            if (it + 3 < n_tiles) load_tile(t0 + 2 * kKvTile, sb);
            compute_tile(1, t0, t0 + kKvTile <= min_vis);
            if (it + 2 < n_tiles) store_tile(0, sa);
            __syncthreads();
        }
    }

    l_run += __shfl_xor(l_run, 32);
    if (tok < 0) return;

    if (a.part_m == nullptr) {
        const float inv = 1.0f / l_run;
        float* orow = a.out + ((int64_t)tok * a.n_q_heads + qh) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * db + 8 * q4 + 4 * hh;
                float4 o;
                o.x = acc[db][4 * q4 + 0] * inv;
                o.y = acc[db][4 * q4 + 1] * inv;
                o.z = acc[db][4 * q4 + 2] * inv;
                o.w = acc[db][4 * q4 + 3] * inv;
                *reinterpret_cast<float4*>(orow + d) = o;
            }
    } else {
        const int64_t pi = ((int64_t)tok * a.n_q_heads + qh) * a.max_splits + split;
        float* prow = a.part_acc + pi * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * db + 8 * q4 + 4 * hh;
                float4 o;
                o.x = acc[db][4 * q4 + 0];
                o.y = acc[db][4 * q4 + 1];
                o.z = acc[db][4 * q4 + 2];
                o.w = acc[db][4 * q4 + 3];
                *reinterpret_cast<float4*>(prow + d) = o;
            }
        if (hh == 0) {
            a.part_m[pi] = m_run;
            a.part_l[pi] = l_run;
        }
    }
}

// One workgroup of D threads per (token, query head).  Combines the splits
// that hold keys visible to the token, loading up to kFast of them in one
// round; padding tokens get a zero row.
template <int D>
__global__ __launch_bounds__(D) void prefill_reduce_kernel(PrefillArgs a) {
    constexpr int kFast = 16;
    const int tok = blockIdx.x;
    const int qh = blockIdx.y;
    const int d = threadIdx.x;
    float* orow = a.out + ((int64_t)tok * a.n_q_heads + qh) * D;
    if (a.token_row[tok] < 0) {
        orow[d] = 0.0f;
        return;
    }
    const int n_vis = min(a.token_kv_len[tok], a.token_pos[tok] + 1);
    const int ns = (n_vis + a.split_tokens - 1) / a.split_tokens;
    const int64_t base = ((int64_t)tok * a.n_q_heads + qh) * a.max_splits;
    float num = 0.0f, den = 0.0f;
    if (ns <= kFast) {
        float pm[kFast], pl[kFast], px[kFast];
#pragma unroll
        for (int s = 0; s < kFast; ++s) {
            if (s < ns) {
                pm[s] = a.part_m[base + s];
                pl[s] = a.part_l[base + s];
                px[s] = a.part_acc[(base + s) * D + d];
            }
        }
        float M = pm[0];
#pragma unroll
        for (int s = 1; s < kFast; ++s)
            if (s < ns) M = fmaxf(M, pm[s]);
#pragma unroll
        for (int s = 0; s < kFast; ++s) {
            if (s < ns) {
                const float f = pm[s] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(pm[s] - M);
                num += f * px[s];
                den += f * pl[s];
            }
        }
    } else {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_m[base + s]);
        for (int s = 0; s < ns; ++s) {
            const float ms = a.part_m[base + s];
            const float f = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
            num += f * a.part_acc[(base + s) * D + d];
            den += f * a.part_l[base + s];
        }
    }
    orow[d] = num / den;
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a, const TileList& tl, int n_items, size_t lds,
                            hipStream_t stream) {
    const int G = a.n_q_heads / a.n_kv_heads;
    const dim3 grid((unsigned)n_items);
    switch (G) {
        case 1: hipLaunchKernelGGL((prefill_kernel<D, 1>), grid, dim3(kThreads), lds, stream, a, tl); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<D, 2>), grid, dim3(kThreads), lds, stream, a, tl); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<D, 4>), grid, dim3(kThreads), lds, stream, a, tl); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<D, 8>), grid, dim3(kThreads), lds, stream, a, tl); break;
        case 16: hipLaunchKernelGGL((prefill_kernel<D, 16>), grid, dim3(kThreads), lds, stream, a, tl); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int prefill_tokens_per_tile(int group) { return kRows / group; }

int prefill_page_table_entries(int split_tokens, int page_size) {
    return (split_tokens + page_size - 1) / page_size + 1;
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillTile* tiles, int n_tiles,
                          int grid_splits, hipStream_t stream) {
    if (n_tiles <= 0) return hipSuccess;
    if (n_tiles > kMaxTilesPerLaunch) return hipErrorInvalidValue;
    TileList tl;
    for (int i = 0; i < n_tiles; ++i) tl.t[i] = tiles[i];
    PrefillArgs b = a;
    b.n_tiles = n_tiles;
    const int n_items = n_tiles * grid_splits * a.n_kv_heads;
    const size_t lds = sizeof(int32_t) * (size_t)prefill_page_table_entries(a.split_tokens, a.page_size);
    if (a.head_dim == 128) return launch_prefill_d<128>(b, tl, n_items, lds, stream);
    return launch_prefill_d<64>(b, tl, n_items, lds, stream);
}

hipError_t launch_prefill_reduce(const PrefillArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_tokens, (unsigned)a.n_q_heads);
    if (a.head_dim == 128)
        hipLaunchKernelGGL(prefill_reduce_kernel<128>, grid, dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL(prefill_reduce_kernel<64>, grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
