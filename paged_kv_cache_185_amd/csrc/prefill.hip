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
// * K and V tiles of 64 keys live in LDS (XOR swizzled in 16-byte units so
//   the MFMA operand reads are free of bank conflicts) and are shared by the
//   8 waves.  They are loaded global -> LDS directly (LDS-direct loads, the
//   swizzle applied on the source side), triple buffered, with no staging
//   registers and no LDS stores; each tile is loaded by the wave group that
//   runs the score half of a phase, between its score MFMAs, three phases
//   before the tile's first use.  MFMA operands are read from LDS a k-step
//   or two ahead of their use.  When the page size is a multiple of 64 a
//   tile never crosses a page: it is one buffer resource (the page's block
//   of the head) and fixed per-thread offsets.  (The unified-span mode
//   stages tiles through registers, double buffered, since its V store
//   zeroes free cells anywhere in a tile.)
// * Both products run on v_mfma_f32_32x32x16_f16 with fp32 accumulation.
//   Scores are computed transposed, S^T = K Q^T (rows = keys, columns =
//   queries): each lane's C registers belong to one query column, so the
//   row max / row sum need one cross-half exchange, and P^T is already in the
//   B-operand layout of O^T = V^T P^T.  The key order of the score rows is
//   permuted (bits 2 and 3 of the row index swapped) so that the 8 keys a lane
//   holds for each P.V k-step are contiguous, which lets the V operand be one
//   16-byte LDS read from the slot-innermost V tile.
// * Q is multiplied by scale*log2(e) and rounded to binary16 once, so scores
//   come out of the MFMA already in the log2 domain, and the score chain
//   starts from -m (the running max), so they come out relative to it; P is
//   rounded to binary16 for the P.V product; row sums and accumulators are
//   fp32.
// * The running maximum is raised only when a new score exceeds it by more
//   than 8 (log2 units): until then P <= 2^8 stays exact enough in binary16
//   and the output rescale (a multiply per accumulator) is skipped.
// * Masking is by select (scores -> -inf), and only on tiles that cross some
//   token's visible end.  V cells at or past the split's visible end (only
//   in its last tile) are zeroed in LDS by the lanes that loaded them before
//   the tile is published, so NaN padding never meets a zero weight.
// * Long KV ranges are split across workgroups.  Each split stores its
//   (m, l, acc) partial; the last split of a (tile, KV head) to finish, found
//   with a device-scope counter, combines them by log-sum-exp in the same
//   launch.
#include <math.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;          // query rows (token x head) per tile
constexpr int kKvTile = kPrefillKvTile;     // 64 keys per iteration
constexpr float kRescaleSlack = 8.0f;       // log2 units the max may lag by
constexpr int kCellPosBits = 22;             // unified span: cell code = seq << 22 | pos
constexpr int kKDepth = 2;                  // K operand k-steps read ahead of the score MFMAs
constexpr int kVDepth = 1;                  // V operand k-steps read ahead of the P.V MFMAs

struct TileList {
    PrefillTile t[kMaxTilesPerLaunch];
};

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Device-scope (all XCDs) 8-byte store, used only for split partials.
__device__ __forceinline__ void store_device2(uint64_t* p, float x, float y) {
    const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS swizzles (16-byte units).  K rows are D*2 bytes; with 64 banks of 4 bytes
// a 16-lane group of 16-byte reads is conflict-free when its 16 chunks cover
// all 256 bytes of the bank range.  The score operand reads 16 different key
// rows at one chunk index, so the chunk is XORed with the key's row index
// within a 256-byte bank line (key & 15 for 256-byte rows; for 128-byte rows
// two keys share a line and (key >> 1) & 7 is used).  V rows (64 keys) are
// 128 bytes, read 16 rows at a time: (d >> 1) & 7.
template <int D>
__device__ __forceinline__ int kswz(int key) {
    return D == 128 ? (key & 15) : ((key >> 1) & 7);
}

__device__ __forceinline__ int vswz(int d) { return (d >> 1) & 7; }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which waits for every outstanding global load (s_waitcnt vmcnt(0))
// and so would drain the K/V prefetch at each tile; the pipeline below only
// communicates through LDS across waves.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt on the vector-memory count only (vmcnt in bits 3:0 and 15:14;
// expcnt, bits 6:4, and lgkmcnt, bits 11:8, left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier of the LDS-direct pipeline.  A release fence on LDS makes
// the compiler wait for every outstanding LDS-direct load (vmcnt(0)) before
// the barrier, which would drain the prefetch each phase.  Here the caller
// waits for exactly the loads the next phase reads (wait_vmcnt), this wave's
// own LDS accesses complete before the barrier (lgkmcnt(0)), and empty asm
// statements with a memory clobber keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void dma_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maxima
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Words 2 and 3 of the raw buffer resources used here: up to 2 GiB of
// records, and data format 32 bit (bits 18:15 of word 3 = 4), other fields 0.
constexpr int kRawRecords = 0x7fffffff;
constexpr int kRawWord3 = 0x00020000;

// K or V tile moved by LDS-direct loads, all of it by one wave group (half
// the workgroup): 16-byte chunks per tile and per thread of the group
template <int D>
struct DmaTile {
    static constexpr int GT = kThreads / 2;
    static constexpr int CH = kKvTile * D / 8;
    static constexpr int PER = CH / GT;
    static_assert(PER * GT == CH, "a tile is a whole number of chunks per thread");
};

// score row i of a 32-key block <-> key offset (bits 2 and 3 swapped)
__device__ __forceinline__ int kappa(int i) {
    return (i & ~0xC) | ((i & 4) << 1) | ((i & 8) >> 1);
}

struct SmemMeta {
    int32_t tok[kRows];
    int32_t last;   // this workgroup combines the tile's splits
};

// Register-staged K/V tiles (unified span only).  Layout of a K tile:
// [key][D/8 chunks], chunk swizzled by kswz(key); of a V tile: [d][8 chunks of
// 8 keys], chunk swizzled by vswz(d).  The paged mode keeps the same tile
// layout in separate LDS arrays filled by LDS-direct loads.
template <int D>
struct SmemStaged {
    u32x4 k[2][kKvTile * D / 8];
    u32x4 v[2][D * kKvTile / 8];
    int32_t kcode[2][kKvTile];  // cell code of each key of a K buffer
};

template <int D>
struct StagingK {
    static constexpr int KC = kKvTile * D / 8 / kThreads;   // 16-byte chunks per thread
    u32x4 k[KC];
    int kcode;   // unified span: cell code of key (tid % 64) of the tile
};

template <int D>
struct StagingV {
    static constexpr int VC = D * kKvTile / 8 / kThreads;   // 16-byte chunks per thread
    u32x4 v[VC];
    int t0;           // first key of the tile held
    uint32_t vlive;   // unified span: bit e = key 8*(tid%8)+e is a written cell
};

// ONE_PAGE: the page size is a multiple of the 64-key tile, so every tile
// lies inside one page and its addresses are one scalar page base plus fixed
// per-thread offsets.
// UNIFIED: the unified-span baseline.  Tiles are runs of consecutive ubatch
// tokens whatever their sequence, every tile scans cells 0..span-1 of the pool
// read as one flat array (page i = cells iP..iP+P-1), and a key is visible to
// a token iff the cell belongs to the token's sequence at a position <= the
// token's; free cells (owner -1) have their V zeroed before the MFMA.
template <int D, int G, bool ONE_PAGE, bool UNIFIED>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a, TileList tl) {
    constexpr int TPW = 32 / G;       // tokens per wave
    constexpr int KS = D / 16;        // k-steps of the score product
    constexpr int DB = D / 32;        // 32-row output blocks
    constexpr int CPR = D / 8;        // 16-byte chunks per K row

    // the grid holds exactly the launch's (tile, split) items, numbered tile
    // by tile, times the KV heads (KV head fastest): no workgroup is empty,
    // so none holds a compute unit that a live one could use
    const int Hkv = a.n_kv_heads;
    const int kvh = blockIdx.x % Hkv;
    const int item = blockIdx.x / Hkv;
    int lo = 0, hi = a.n_tiles - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tl.t[mid].item0 <= item) lo = mid;
        else hi = mid - 1;
    }
    const int tile_idx = lo;
    const PrefillTile tile = tl.t[tile_idx];
    const int split = item - tile.item0;
    if (split >= tile.n_splits) return;
    const int kv_begin = split * tile.split_len;
    const int kv_end = min(tile.kv_end, kv_begin + tile.split_len);

    __shared__ SmemMeta sm;
    __shared__ SmemStaged<D> ss;   // referenced by the unified-span path only
    // paged mode: triple-buffered K and V tiles, filled by LDS-direct loads
    constexpr int TCH = DmaTile<D>::CH;
    __shared__ u32x4 kt0[TCH], kt1[TCH], kt2[TCH], vt0[TCH], vt1[TCH], vt2[TCH];
    extern __shared__ int32_t sm_pages[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int hh = lane >> 5;
    const int P = a.page_size;

    // ---- this split's page ids -> LDS (loaded first: the in-order vmcnt
    // accounting then lets the Q loads below stay in flight across the
    // barrier), and this lane's query column: tile row (wave*32 + col) is
    // token slot row/G, head row%G.  A dense tile's tokens are first..last,
    // so its metadata and Q loads start at once; otherwise wave 0 finds the
    // tile's tokens with a ballot scan of token_row[first..last].
    const int sh = a.page_shift;
    const int page_base = kv_begin >> sh;
    const int32_t* bt = a.block_tables + (int64_t)tile.row * a.max_pages;
    const int n_pages = ((kv_end - 1) >> sh) - page_base + 1;
    // unified span: page i of the span is pool page i
    const int pt0 = UNIFIED ? page_base + tid : (tid < n_pages ? bt[page_base + tid] : 0);
    // the first tile's page (entry 0), read by every lane at one address
    const int page0 = UNIFIED ? page_base : bt[page_base];
    const int ti = wave * TPW + col / G;
    const int hq = col % G;
    const int qh = kvh * G + hq;
    int tok = -1;
    int tok_kv_len = 0, tok_pos = 0, tok_seq = -1;
    int n_vis = 0;   // keys this lane's query token sees
    float4 qraw[2 * KS];
    auto load_token = [&]() __attribute__((always_inline)) {
        const int t = tok >= 0 ? tok : 0;
        if constexpr (UNIFIED)
            tok_seq = tok >= 0 ? a.token_row[t] : -1;
        else
            tok_kv_len = a.token_kv_len[t];
        tok_pos = a.token_pos[t];
        const float* qrow = a.q + ((int64_t)t * a.n_q_heads + qh) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int d0 = 16 * ks + 8 * hh;
            qraw[2 * ks] = *reinterpret_cast<const float4*>(qrow + d0);
            qraw[2 * ks + 1] = *reinterpret_cast<const float4*>(qrow + d0 + 4);
        }
    };
    if (tile.dense) {
        tok = ti < tile.count ? tile.first + ti : -1;
        load_token();
    } else if (wave == 0) {
        // eight 64-entry chunks of token_row in flight per round
        int found = 0;
        for (int base = tile.first; base <= tile.last && found < tile.count; base += 512) {
            int rw[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = base + 64 * k + lane;
                rw[k] = i <= tile.last ? a.token_row[i] : -1;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = base + 64 * k + lane;
                const bool hit = i <= tile.last && rw[k] == tile.row;
                const uint64_t mask = __ballot(hit);
                const int before = __popcll(mask & ((1ull << lane) - 1ull));
                if (hit && found + before < tile.count) sm.tok[found + before] = i;
                found += __popcll(mask);
            }
        }
    }
    if (tid < n_pages) sm_pages[tid] = pt0;
    for (int i = tid + kThreads; i < n_pages; i += kThreads) sm_pages[i] = UNIFIED ? page_base + i : bt[page_base + i];
    __syncthreads();
    // a tile found by the scan: its tokens' metadata and Q are loaded once
    // the first K/V loads are out
    auto load_scanned_token = [&]() __attribute__((always_inline)) {
        if (!tile.dense) {
            tok = ti < tile.count ? sm.tok[ti] : -1;
            load_token();
        }
    };

    u32x4 qb[KS];   // Q operands, made once the first tile's loads are out

    const uint16_t* kc = a.k_cache;
    const uint16_t* vc = a.v_cache;

    // ---- unified span: global -> registers for one KV tile starting at key
    // t0 (the paged mode loads tiles straight into LDS, below).  Thread
    // tid moves the K chunks (key, c) = (id / CPR, id % CPR) and the V chunks
    // (d, c) = (id / 8, id % 8) of id = tid + kThreads*i; everything but the
    // page lookup is fixed per thread.  Loads and stores are branch-free
    // (tiles past the end are clamped onto the last one, the V mask is an
    // unconditional AND at store time), so the in-order vmcnt accounting is
    // the same on every path and a store waits only for its own tile.
    const int64_t page_elems = (int64_t)Hkv * P * D;   // one page of one cache, all heads
    const int k_head_off = kvh * P * D;
    const int last_t0 = kv_begin + ((kv_end - kv_begin - 1) / kKvTile) * kKvTile;
    // per-thread element offsets of the K chunks (key, c) and V chunks (d, c)
    // inside one tile when it lies in one page
    int koff[StagingK<D>::KC], voff[StagingV<D>::VC];
#pragma unroll
    for (int i = 0; i < StagingK<D>::KC; ++i) {
        const int id = tid + kThreads * i;
        koff[i] = (id / CPR) * D + 8 * (id % CPR);
    }
    // (one-page tiles: P is a multiple of 64, so V slot blocks hold 32 slots
    // and the tile's 64 keys are two consecutive blocks)
#pragma unroll
    for (int i = 0; i < StagingV<D>::VC; ++i) {
        const int id = tid + kThreads * i;
        const int c = id & 7;
        voff[i] = (c >> 2) * (kVSlotTile * D) + (id >> 3) * kVSlotTile + 8 * (c & 3);
    }
    auto load_meta_k = [&](int t0, StagingK<D>& st) __attribute__((always_inline)) {
        if constexpr (UNIFIED) {
            // every lane loads (clamped, so the loads are unconditional); lanes
            // 0..63 of the workgroup store key (tid % 64)'s owner and position
            const int t = t0 + (tid & (kKvTile - 1));
            const int tc = min(t, kv_end - 1);
            const int sq = a.cell_seq[tc];
            const int ps = a.cell_pos[tc];
            st.kcode = (t < kv_end && sq >= 0) ? (sq << kCellPosBits) + ps : -1;
        }
    };
    auto load_meta_v = [&](int t0, StagingV<D>& st) __attribute__((always_inline)) {
        if constexpr (UNIFIED) {
            // keys 8c..8c+7 of this thread's V chunks: live iff inside the
            // split and written (owner >= 0)
            const int tb = t0 + 8 * (tid & 7);
            uint32_t live = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sq = a.cell_seq[min(tb + e, kv_end - 1)];
                live |= (tb + e < kv_end && sq >= 0) ? (1u << e) : 0u;
            }
            st.vlive = live;
        }
    };
    // one-page tiles.  In the tile that crosses the split's visible end (the
    // split's last), K rows past the end are loaded from the last visible row
    // and V 8-slot runs past it from the run holding the last visible slot,
    // so no cell past the end is read except the slots that share that run's
    // 16-byte vector; those scores are masked and those V halves zeroed at
    // store.  The branch is uniform and both arms issue the same loads.
    auto load_k_page = [&](int t0, int page, StagingK<D>& st) __attribute__((always_inline)) {
        load_meta_k(t0, st);
        const uint16_t* kb = kc + page * page_elems + (k_head_off + (t0 & (P - 1)) * D);
        if (t0 + kKvTile <= kv_end) {
#pragma unroll
            for (int i = 0; i < StagingK<D>::KC; ++i) st.k[i] = *reinterpret_cast<const u32x4*>(kb + koff[i]);
        } else {
            const int kmax = kv_end - 1 - t0;
#pragma unroll
            for (int i = 0; i < StagingK<D>::KC; ++i) {
                const int id = tid + kThreads * i;
                st.k[i] = *reinterpret_cast<const u32x4*>(kb + min(id / CPR, kmax) * D + 8 * (id % CPR));
            }
        }
    };
    auto load_v_page = [&](int t0, int page, StagingV<D>& st) __attribute__((always_inline)) {
        st.t0 = t0;
        load_meta_v(t0, st);
        const uint16_t* vb = vc + page * page_elems + (k_head_off + (int64_t)(t0 & (P - 1)) * D);
        if (t0 + kKvTile <= kv_end) {
#pragma unroll
            for (int i = 0; i < StagingV<D>::VC; ++i) st.v[i] = *reinterpret_cast<const u32x4*>(vb + voff[i]);
        } else {
            const int c = min(tid & 7, (kv_end - 1 - t0) >> 3);
#pragma unroll
            for (int i = 0; i < StagingV<D>::VC; ++i) {
                const int d = (tid + kThreads * i) >> 3;
                st.v[i] = *reinterpret_cast<const u32x4*>(vb + (c >> 2) * (kVSlotTile * D) + d * kVSlotTile +
                                                          8 * (c & 3));
            }
        }
    };
    auto load_k = [&](int t0_req, StagingK<D>& st) __attribute__((always_inline)) {
        const int t0 = min(t0_req, last_t0);
        if constexpr (!ONE_PAGE) load_meta_k(t0, st);
        if constexpr (ONE_PAGE) {
            load_k_page(t0, __builtin_amdgcn_readfirstlane(sm_pages[(t0 >> sh) - page_base]), st);
        } else {
#pragma unroll
            for (int i = 0; i < StagingK<D>::KC; ++i) {
                const int id = tid + kThreads * i;
                const int key = id / CPR;
                const int c = id % CPR;
                const int t = min(t0 + key, kv_end - 1);
                const int page = sm_pages[(t >> sh) - page_base];
                st.k[i] = *reinterpret_cast<const u32x4*>(
                    kc + page * page_elems + (k_head_off + (t & (P - 1)) * D + 8 * c));
            }
        }
    };
    auto load_v = [&](int t0_req, StagingV<D>& st) __attribute__((always_inline)) {
        const int t0 = min(t0_req, last_t0);
        st.t0 = t0;
        if constexpr (!ONE_PAGE) load_meta_v(t0, st);
        if constexpr (ONE_PAGE) {
            load_v_page(t0, __builtin_amdgcn_readfirstlane(sm_pages[(t0 >> sh) - page_base]), st);
        } else {
            const int c = tid & 7;
            const int tb = t0 + 8 * c;
            const int tv = tb < kv_end ? tb : ((kv_end - 1) & ~7);
            const int vpage = sm_pages[(tv >> sh) - page_base];
            // keys tv..tv+7 (8-aligned) lie in one V slot block of VT slots
            const int VT = v_slot_tile(P);
            const int vslot = tv & (P - 1);
            const uint16_t* vbase = vc + vpage * page_elems +
                                    (k_head_off + (int64_t)(vslot & ~(VT - 1)) * D + (vslot & (VT - 1)));
#pragma unroll
            for (int i = 0; i < StagingV<D>::VC; ++i) {
                const int d = (tid + kThreads * i) >> 3;
                st.v[i] = *reinterpret_cast<const u32x4*>(vbase + d * VT);
            }
        }
    };
    auto store_k = [&](int buf, StagingK<D>& st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < StagingK<D>::KC; ++i) {
            const int id = tid + kThreads * i;
            const int key = id / CPR;
            const int c = id % CPR;
            ss.k[buf][key * CPR + (c ^ kswz<D>(key))] = st.k[i];
        }
        if constexpr (UNIFIED) {
            if (tid < kKvTile) ss.kcode[buf][tid] = st.kcode;
        }
    };
    auto store_v = [&](int buf, StagingV<D>& st) __attribute__((always_inline)) {
        {
            // zero the V halves of free cells and of keys past the split
            uint32_t mk[4];
#pragma unroll
            for (int w = 0; w < 4; ++w)
                mk[w] = ((st.vlive >> (2 * w)) & 1u ? 0x0000ffffu : 0u) |
                        ((st.vlive >> (2 * w + 1)) & 1u ? 0xffff0000u : 0u);
#pragma unroll
            for (int i = 0; i < StagingV<D>::VC; ++i)
#pragma unroll
                for (int w = 0; w < 4; ++w) st.v[i][w] &= mk[w];
        }
#pragma unroll
        for (int i = 0; i < StagingV<D>::VC; ++i) {
            const int id = tid + kThreads * i;
            const int d = id >> 3;
            const int c = id & 7;
            ss.v[buf][d * 8 + (c ^ vswz(d))] = st.v[i];
        }
    };

    // ---- paged mode: LDS-direct tile loads, each tile by the four waves of
    // one group.  One global_load_lds_dwordx4 moves 16 bytes per lane into 64
    // consecutive 16-byte LDS chunks at a wave-uniform base, so the swizzle is
    // applied on the source side: LDS chunk p = tg + GT*i of a tile (tg = the
    // thread's index in its group) receives the logical chunk that the
    // swizzled layout keeps at p.  The chunk column a lane fetches is the same
    // for every i; only the key (K) or value row (V) moves with i.
    constexpr int GT = DmaTile<D>::GT;
    const int tg = tid & (GT - 1);
    const int ck = (tg % CPR) ^ kswz<D>(tg / CPR);   // K: chunk of the key row
    const int cv = (tg & 7) ^ vswz(tg >> 3);          // V: 8-key run of the value row
    const int wbase = (__builtin_amdgcn_readfirstlane(wave) & 3) * 64;
    auto dma16 = [&](const uint16_t* src, u32x4* dst) __attribute__((always_inline)) {
        __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    };
    // one-page tiles: the tile's K or V block of this head as a buffer
    // resource (built once per tile in scalar registers), and one load of it
    // with a per-lane 32-bit byte offset
    auto tile_rsrc = [&](const uint16_t* cache, int t0) __attribute__((always_inline)) {
        const int page = __builtin_amdgcn_readfirstlane(sm_pages[(t0 >> sh) - page_base]);
        const uint16_t* base = cache + page * page_elems + (k_head_off + (int64_t)(t0 & (P - 1)) * D);
        return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, kRawRecords, kRawWord3);
    };
    auto dma_kb = [&](u32x4* dst, __amdgpu_buffer_rsrc_t r, int t0, int i) __attribute__((always_inline)) {
        const int key = min(tg / CPR + (GT / CPR) * i, min(kKvTile - 1, kv_end - 1 - t0));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + GT * i + wbase), 16,
                                                 (key * D + 8 * ck) * 2, 0, 0, 0);
    };
    auto dma_vb = [&](u32x4* dst, __amdgpu_buffer_rsrc_t r, int t0, int i) __attribute__((always_inline)) {
        const int c = min(cv, (kv_end - 1 - t0) >> 3);
        const int d = (tg >> 3) + (GT / 8) * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + GT * i + wbase), 16,
                                                 ((c >> 2) * (kVSlotTile * D) + d * kVSlotTile + 8 * (c & 3)) * 2, 0, 0, 0);
    };
    auto dma_k = [&](u32x4* dst, int t0_req) __attribute__((always_inline)) {
        const int t0 = min(t0_req, last_t0);
        // rows at or past the visible end are fetched from the last visible
        // row (their scores are masked)
        const int kmax = min(kKvTile - 1, kv_end - 1 - t0);
        if constexpr (ONE_PAGE) {
            const int page = __builtin_amdgcn_readfirstlane(sm_pages[(t0 >> sh) - page_base]);
            const uint16_t* kb = kc + page * page_elems + (k_head_off + (t0 & (P - 1)) * D + 8 * ck);
#pragma unroll
            for (int i = 0; i < DmaTile<D>::PER; ++i) {
                const int key = min(tg / CPR + (GT / CPR) * i, kmax);
                dma16(kb + key * D, dst + GT * i + wbase);
            }
        } else {
#pragma unroll
            for (int i = 0; i < DmaTile<D>::PER; ++i) {
                const int t = t0 + min(tg / CPR + (GT / CPR) * i, kmax);
                const int page = sm_pages[(t >> sh) - page_base];
                dma16(kc + page * page_elems + (k_head_off + (t & (P - 1)) * D + 8 * ck), dst + GT * i + wbase);
            }
        }
    };
    auto dma_v = [&](u32x4* dst, int t0_req) __attribute__((always_inline)) {
        const int t0 = min(t0_req, last_t0);
        // 8-slot runs at or past the visible end are fetched from the run
        // holding the last visible slot; fix_v_tail zeroes what lies past it
        const int c = min(cv, (kv_end - 1 - t0) >> 3);
        if constexpr (ONE_PAGE) {
            // V slot blocks of kVSlotTile slots: the tile is two whole blocks
            const int page = __builtin_amdgcn_readfirstlane(sm_pages[(t0 >> sh) - page_base]);
            const uint16_t* vb = vc + page * page_elems +
                                 (k_head_off + (int64_t)(t0 & (P - 1)) * D + (c >> 2) * (kVSlotTile * D) +
                                  8 * (c & 3));
#pragma unroll
            for (int i = 0; i < DmaTile<D>::PER; ++i) {
                const int d = (tg >> 3) + (GT / 8) * i;
                dma16(vb + d * kVSlotTile, dst + GT * i + wbase);
            }
        } else {
            // keys tb..tb+7 (8-aligned, below kv_end) lie in one slot block
            const int tb = t0 + 8 * c;
            const int vpage = sm_pages[(tb >> sh) - page_base];
            const int VT = v_slot_tile(P);
            const int vslot = tb & (P - 1);
            const uint16_t* vbase = vc + vpage * page_elems +
                                    (k_head_off + (int64_t)(vslot & ~(VT - 1)) * D + (vslot & (VT - 1)));
#pragma unroll
            for (int i = 0; i < DmaTile<D>::PER; ++i) {
                const int d = (tg >> 3) + (GT / 8) * i;
                dma16(vbase + d * VT, dst + GT * i + wbase);
            }
        }
    };
    // Zero the V halves of keys at or past the visible end in the chunks this
    // lane loaded into the split's last V tile, once its own loads are done
    // and before the barrier that publishes the tile.
    auto fix_v_tail = [&](u32x4* vt, int t0) __attribute__((always_inline)) {
        const int nvalid = kv_end - (t0 + 8 * cv);
        if (nvalid < 8) {
            uint32_t mk[4];
#pragma unroll
            for (int w = 0; w < 4; ++w)
                mk[w] = (2 * w < nvalid ? 0x0000ffffu : 0u) | (2 * w + 1 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
            for (int i = 0; i < DmaTile<D>::PER; ++i) {
                u32x4 x = vt[GT * i + tg];
#pragma unroll
                for (int w = 0; w < 4; ++w) x[w] &= mk[w];
                vt[GT * i + tg] = x;
            }
        }
    };

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
    f32x16 s[2];   // scores of the tile between its two phases, minus m_use
    float m_use = 0.0f;   // running max the scores are taken relative to (0 while none seen)
    // -m_use in all 16 rows (every row of a lane's accumulator block belongs
    // to the lane's query column): the score MFMA chain starts from it, so
    // scores come out already relative to the running max and the softmax
    // needs no subtraction
    f32x16 negm;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = 0.0f;

    // S^T = K Q^T for the 64 keys t0..t0+63 of K tile `kt`, then the first
    // half of the online softmax: the mask (`full`, uniform, says every query
    // column sees all 64 keys), the row maximum and the lazy rescale.  These
    // sit in the score half of the ping-pong (measured 1.4% faster than in the
    // softmax half when tiles went through registers).  With the tile loads
    // this half is the longer one of a phase: moving the exps of the first one
    // or two P.V k-steps into it is 1.5% and 3% slower.  K operands are read
    // from LDS two k-steps ahead of their MFMAs, and the two 32-key blocks
    // alternate so consecutive MFMAs are independent.  mid(ks) runs after
    // k-step ks (the phase's tile loads go there).
    auto qk = [&](const u32x4* kt, const int32_t* kcode, int t0, bool full, auto&& mid) __attribute__((always_inline)) {
        const int krow0 = kappa(col);
        const int krow1 = 32 + kappa(col);
        auto kread = [&](int ks, int krow) __attribute__((always_inline)) {
            const int c = 2 * ks + hh;
            return kt[krow * CPR + (c ^ kswz<D>(krow))];
        };
        // ring of kKDepth+1 k-steps of operands, kKDepth in flight
        constexpr int R = kKDepth + 1;
        u32x4 ka[R], kb1[R];
#pragma unroll
        for (int ks = 0; ks < kKDepth; ++ks) {
            ka[ks] = kread(ks, krow0);
            kb1[ks] = kread(ks, krow1);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + kKDepth < KS) {
                ka[(ks + kKDepth) % R] = kread(ks + kKDepth, krow0);
                kb1[(ks + kKDepth) % R] = kread(ks + kKDepth, krow1);
            }
            // keep the scheduler from sinking the reads back to their use
            __builtin_amdgcn_sched_barrier(0);
            if (ks == 0) {
                s[0] = mfma32(ka[0], qb[0], negm);
                s[1] = mfma32(kb1[0], qb[0], negm);
            } else {
                s[0] = mfma32(ka[ks % R], qb[ks], s[0]);
                s[1] = mfma32(kb1[ks % R], qb[ks], s[1]);
            }
            __builtin_amdgcn_sched_barrier(0);
            mid(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (UNIFIED) {
            // visible iff the cell is this token's sequence at a position not
            // after the token's: its code lies in [seq << bits, (seq << bits) +
            // pos] (free cells are -1); the lane's keys come in runs of 8
            const uint32_t lo = (uint32_t)(tok_seq << kCellPosBits);
            const uint32_t span_hi = tok_seq >= 0 ? (uint32_t)tok_pos : 0u;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int k0 = 32 * kb + 16 * j + 8 * hh;
                    const int4 c0 = *reinterpret_cast<const int4*>(&kcode[k0]);
                    const int4 c1 = *reinterpret_cast<const int4*>(&kcode[k0 + 4]);
                    const int cd[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool vis = tok_seq >= 0 && cd[e] >= 0 && (uint32_t)cd[e] - lo <= span_hi;
                        s[kb][8 * j + e] = vis ? s[kb][8 * j + e] : -INFINITY;
                    }
                }
        } else if (!full) {
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
        {
            // the other half-wave holds the same query column's other keys:
            // one of the two swap results is mx itself, the other its partner
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                             false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        mx += m_use;   // the tile's maximum in absolute terms
        // raise the running max only when the new one is well above it; then
        // rescale the accumulators and re-base this tile's scores and the
        // chain start on the new max
        const bool raise = mx > m_run + kRescaleSlack;
        if (__ballot(raise)) {
            const float m_new = raise ? mx : m_run;
            const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= alpha;
            m_run = m_new;
            const float m_use_new = m_run == -INFINITY ? 0.0f : m_run;
            const float shift = m_use - m_use_new;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] += shift;
#pragma unroll
            for (int r = 0; r < 16; ++r) negm[r] = -m_use_new;
            m_use = m_use_new;
        }
    };

    // Second half of the online softmax of the scores (P = exp2(s), the
    // scores being relative to the running max already; row sums) and
    // O^T += V^T P^T with V tile `vt`.
    auto smpv = [&](const u32x4* vt) __attribute__((always_inline)) {
        // raised wave priority: this wave's instructions go first when both
        // waves of a SIMD can issue (measured 1% faster, with register-staged
        // and with LDS-direct tiles; priority on the score MFMAs instead was
        // 2.5% slower)
        __builtin_amdgcn_s_setprio(1);
        // 16 keys per k-step: P is made just before its MFMAs and the V
        // operands of the next k-step are read from LDS meanwhile
        auto vread = [&](int ks, int db) __attribute__((always_inline)) {
            const int c = 2 * ks + hh;
            const int d = 32 * db + col;
            return vt[d * 8 + (c ^ vswz(d))];
        };
        // ring of kVDepth+1 k-steps of V operands, kVDepth in flight
        constexpr int RV = kVDepth + 1;
        u32x4 vop[RV][DB];
#pragma unroll
        for (int ks = 0; ks < kVDepth; ++ks)
#pragma unroll
            for (int db = 0; db < DB; ++db) vop[ks][db] = vread(ks, db);
        // the row sum adds the binary16 P the MFMA consumes, two per dot2
        const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        float psum[2] = {0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + kVDepth < 4) {
#pragma unroll
                for (int db = 0; db < DB; ++db) vop[(ks + kVDepth) % RV][db] = vread(ks + kVDepth, db);
            }
            f16x8 p;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                p[e] = (_Float16)__builtin_amdgcn_exp2f(s[ks >> 1][8 * (ks & 1) + e]);
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const f16x2 pp = {p[e], p[e + 1]};
                psum[(e >> 1) & 1] = __builtin_amdgcn_fdot2(pp, ones, psum[(e >> 1) & 1], false);
            }
            const u32x4 pb = __builtin_bit_cast(u32x4, p);
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] = mfma32(vop[ks % RV][db], pb, acc[db]);
        }
        l_run += psum[0] + psum[1];
        __builtin_amdgcn_s_setprio(0);
    };

    // smallest visible length over the tile's tokens (from the plan): tiles
    // ending at or before it need no mask
    const int min_vis = UNIFIED ? 0 : min(tile.min_vis, kv_end);
    const int n_tiles = (kv_end - kv_begin + kKvTile - 1) / kKvTile;

    // ---- main loop: two wave groups in ping-pong.  Waves 0-3 (group A) and
    // 4-7 (group B) share the SIMDs pairwise; in every phase one group runs
    // the score MFMAs, mask and row maximum of a tile while the other runs
    // the exps and P.V MFMAs of the previous one, so matrix and vector work
    // of the two waves on a SIMD overlap.  Tile j: A does QK(j) in phase 2j
    // and softmax+PV(j) in phase 2j+1, B one phase later, so K(j) is read in
    // phases 2j and 2j+1 and V(j) in phases 2j+1 and 2j+2; 2*n_tiles+1
    // phases in all, each ended by a barrier.  Each group runs its own loop
    // (same loads and barriers per phase) so that register lifetimes stay
    // simple for the compiler.
    const int wgroup = __builtin_amdgcn_readfirstlane(wave >> 2);
    // Q times scale*log2(e), rounded to binary16: scores come out of the MFMA
    // in the log2 domain
    auto make_q = [&]() __attribute__((always_inline)) {
        const float qs = tok >= 0 ? a.scale_log2 : 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 x0 = qraw[2 * ks];
            const float4 x1 = qraw[2 * ks + 1];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            f16x8 h;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (_Float16)(xs[e] * qs);
            qb[ks] = __builtin_bit_cast(u32x4, h);
        }
    };

    if constexpr (UNIFIED) {
        // Unified span: tiles go global -> registers -> LDS (the V store
        // zeroes free cells), double buffered; global loads run two phases
        // (one tile) ahead of their LDS stores and are clamped onto the last
        // tile past the end, so every phase issues the same loads.  K(j) is
        // stored in the phase before its first use, V(j) likewise.
        load_scanned_token();
        StagingK<D> stk;
        StagingV<D> stv;
        if constexpr (ONE_PAGE) {
            load_k_page(kv_begin, page0, stk);
            load_v_page(kv_begin, page0, stv);
        } else {
            load_k(kv_begin, stk);
            load_v(kv_begin, stv);
        }
        make_q();
        n_vis = tok >= 0 ? min(tok_kv_len, tok_pos + 1) : 0;
        store_k(0, stk);
        load_k(kv_begin + kKvTile, stk);
        __syncthreads();
        if (wgroup == 0) {
            for (int j = 0; j < n_tiles; ++j) {
                const int tj = kv_begin + j * kKvTile;
                // phase 2j: V(j) -> LDS; QK(j)
                store_v(j & 1, stv);
                load_v(tj + kKvTile, stv);
                qk(ss.k[j & 1], ss.kcode[j & 1], tj, false, [](int) {});
                lds_barrier();
                // phase 2j+1: K(j+1) -> LDS; softmax+PV(j)
                store_k((j + 1) & 1, stk);
                load_k(tj + 2 * kKvTile, stk);
                smpv(ss.v[j & 1]);
                lds_barrier();
            }
            // phase 2n: the other group's last softmax+PV
            store_v(n_tiles & 1, stv);
            lds_barrier();
        } else {
            // phase 0: the other group's first QK
            store_v(0, stv);
            load_v(kv_begin + kKvTile, stv);
            lds_barrier();
            for (int j = 0; j < n_tiles; ++j) {
                const int tj = kv_begin + j * kKvTile;
                // phase 2j+1: K(j+1) -> LDS; QK(j)
                store_k((j + 1) & 1, stk);
                load_k(tj + 2 * kKvTile, stk);
                qk(ss.k[j & 1], ss.kcode[j & 1], tj, false, [](int) {});
                lds_barrier();
                // phase 2j+2: V(j+1) -> LDS; softmax+PV(j)
                store_v((j + 1) & 1, stv);
                load_v(tj + 2 * kKvTile, stv);
                smpv(ss.v[j & 1]);
                lds_barrier();
            }
        }
    } else if (n_tiles > 0) {
        // Paged mode: tiles go global -> LDS directly (global_load_lds), K and
        // V triple buffered (tile m in buffer m % 3), so no staging registers
        // and no LDS stores.  Each group loads one kind of tile during its
        // score phases, so the softmax and P.V waves issue no loads: group A
        // loads K(j+2) in phase 2j, during QK(j), and group B loads V(j+2) in
        // phase 2j+1, during its QK(j).  A compute unit's vector-memory path
        // takes one of these 1 KiB loads every ~15-19 cycles, so a wave that
        // issues into a burst of its neighbours' loads waits; with one-page
        // tiles the loads go out one after every other score k-step (a buffer
        // resource per tile, one 32-bit offset per lane and load), otherwise
        // after the score MFMAs.  A tile is
        // first read four phases after its loads are issued.  At the end of
        // its softmax phase a group waits for its own tile loaded two phases
        // before the latest (one tile's loads may stay in flight), and the
        // barrier then publishes it to every wave: A waits for K(j+1) at the
        // end of phase 2j+1, B for V(j+1) at the end of phase 2j+2.  A load
        // overwrites the buffer of tile m-3, whose last reader ran in an
        // earlier phase.  Loads past the last tile are clamped onto it (never
        // read), so every pass issues the same loads and the wait count is
        // the same everywhere.  The loop is unrolled by three so that every
        // buffer is a distinct LDS variable at every access: the compiler
        // then orders an operand read only after the loads into its own
        // buffer.  Each pass runs all three steps (up to two past the last
        // tile only load and take their barriers): exits inside the unrolled
        // body made the compiler drain every load (vmcnt(0)) at the top of
        // each pass.
        auto kt = [&](auto bc) __attribute__((always_inline)) -> u32x4* {
            if constexpr (decltype(bc)::value == 0) return kt0;
            else if constexpr (decltype(bc)::value == 1) return kt1;
            else return kt2;
        };
        auto vt = [&](auto bc) __attribute__((always_inline)) -> u32x4* {
            if constexpr (decltype(bc)::value == 0) return vt0;
            else if constexpr (decltype(bc)::value == 1) return vt1;
            else return vt2;
        };
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        using B2 = std::integral_constant<int, 2>;
        // end of a softmax phase: this wave's loads but the latest tile's
        // are complete
        auto phase_wait = [&]() __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<DmaTile<D>::PER>();
            __builtin_amdgcn_sched_barrier(0);
        };
        // the first tile, the token metadata and Q (a tile found by the scan;
        // a contiguous tile loaded them before the page table), then the
        // second tile: the in-order wait for Q in make_q leaves the second
        // tile's loads in flight.  Each path makes Q on its own, so that the
        // compiler counts its own loads exactly instead of draining them all
        // where the paths join.
        if (wgroup == 0) dma_k(kt0, kv_begin);
        else dma_v(vt0, kv_begin);
        auto second_tile = [&]() __attribute__((always_inline)) {
            if (wgroup == 0) dma_k(kt1, kv_begin + kKvTile);
            else dma_v(vt1, kv_begin + kKvTile);
        };
        if (!tile.dense) {
            load_scanned_token();
            second_tile();
            make_q();
        } else {
            second_tile();
            make_q();
        }
        n_vis = tok >= 0 ? min(tok_kv_len, tok_pos + 1) : 0;
        if (wgroup == 0) {
            phase_wait();   // K(0)
            dma_barrier();
            auto a_tile = [&](auto bc, int j) __attribute__((always_inline)) {
                constexpr int B = decltype(bc)::value;
                using Bn2 = std::integral_constant<int, (B + 2) % 3>;
                const int tj = kv_begin + j * kKvTile;
                // phase 2j: QK(j); load K(j+2) into K(j-1)'s buffer
                constexpr int STEP = KS / DmaTile<D>::PER;
                if constexpr (ONE_PAGE) {
                    const int tq = min(tj + 2 * kKvTile, last_t0);
                    const auto rk = tile_rsrc(kc, tq);
                    if (j < n_tiles) {
                        qk(kt(bc), nullptr, tj, tj + kKvTile <= min_vis, [&](int ks) __attribute__((always_inline)) {
                            if (ks % STEP == 0) dma_kb(kt(Bn2{}), rk, tq, ks / STEP);
                        });
                    } else {
#pragma unroll
                        for (int i = 0; i < DmaTile<D>::PER; ++i) dma_kb(kt(Bn2{}), rk, tq, i);
                    }
                } else {
                    if (j < n_tiles) qk(kt(bc), nullptr, tj, tj + kKvTile <= min_vis, [](int) {});
                    __builtin_amdgcn_sched_barrier(0);
                    dma_k(kt(Bn2{}), tj + 2 * kKvTile);
                }
                dma_barrier();
                // phase 2j+1: softmax+PV(j)
                if (j < n_tiles) smpv(vt(bc));
                phase_wait();   // K(j+1)
                dma_barrier();
            };
            for (int j = 0; j < n_tiles; j += 3) {
                a_tile(B0{}, j);
                a_tile(B1{}, j + 1);
                a_tile(B2{}, j + 2);
            }
            // phase 2n: the other group's last softmax+PV
            dma_barrier();
        } else {
            dma_barrier();
            // phase 0: the other group's first QK
            phase_wait();   // V(0)
            if (n_tiles == 1) fix_v_tail(vt0, kv_begin);
            dma_barrier();
            auto b_tile = [&](auto bc, int j) __attribute__((always_inline)) {
                constexpr int B = decltype(bc)::value;
                using Bn1 = std::integral_constant<int, (B + 1) % 3>;
                using Bn2 = std::integral_constant<int, (B + 2) % 3>;
                const int tj = kv_begin + j * kKvTile;
                // phase 2j+1: QK(j); load V(j+2) into V(j-1)'s buffer
                constexpr int STEP = KS / DmaTile<D>::PER;
                if constexpr (ONE_PAGE) {
                    const int tq = min(tj + 2 * kKvTile, last_t0);
                    const auto rv = tile_rsrc(vc, tq);
                    if (j < n_tiles) {
                        qk(kt(bc), nullptr, tj, tj + kKvTile <= min_vis, [&](int ks) __attribute__((always_inline)) {
                            if (ks % STEP == 0) dma_vb(vt(Bn2{}), rv, tq, ks / STEP);
                        });
                    } else {
#pragma unroll
                        for (int i = 0; i < DmaTile<D>::PER; ++i) dma_vb(vt(Bn2{}), rv, tq, i);
                    }
                } else {
                    if (j < n_tiles) qk(kt(bc), nullptr, tj, tj + kKvTile <= min_vis, [](int) {});
                    __builtin_amdgcn_sched_barrier(0);
                    dma_v(vt(Bn2{}), tj + 2 * kKvTile);
                }
                dma_barrier();
                // phase 2j+2: softmax+PV(j)
                if (j < n_tiles) smpv(vt(bc));
                phase_wait();   // V(j+1)
                if (j + 1 == n_tiles - 1) fix_v_tail(vt(Bn1{}), tj + kKvTile);
                dma_barrier();
            };
            for (int j = 0; j < n_tiles; j += 3) {
                b_tile(B0{}, j);
                b_tile(B1{}, j + 1);
                b_tile(B2{}, j + 2);
            }
        }
        // no load may still be writing LDS when the workgroup moves on
        wait_vmcnt<0>();
    } else {
        load_scanned_token();   // no keys: the rows are written as zeros
    }

    // ---- epilogue.  l_run holds this half-wave's keys only; the column's
    // total adds the partner half's (one of the two swap results is the
    // lane's own value, the other its partner's).
    auto pair_sum = [](float x) __attribute__((always_inline)) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    };
    auto write_out = [&](float l_tot) __attribute__((always_inline)) {
        // a token that sees no key (unified span: no cell of its sequence up
        // to its position) gets a zero row
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
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
    };
    if (tile.n_splits == 1) {
        const float l_tot = pair_sum(l_run);
        if (tok >= 0) write_out(l_tot);
        return;
    }

    // ---- split tile: fused log-sum-exp combine.  Each split stores its
    // partial as the normalised output o = acc / l rounded to binary16 (its
    // magnitude is bounded by |V|, so the rounding costs about 2^-11
    // relative, and it halves the bytes written and read back) plus (m, l)
    // in fp32, in the lanes' register order, with device-scope stores
    // (written through past the per-XCD L2s); waits until they are
    // acknowledged, and bumps the (tile, KV head) counter.  The split that
    // brings it to n_splits reads the others' partials with device-scope
    // loads and forms sum(w l o) / sum(w l), w = exp2(m - max m), folding the
    // splits in ascending order; it writes the output and zeroes the counter.
    constexpr int NP = 2 * DB;   // 16-byte pieces (8 halves) of binary16 output per lane
    const int64_t grp = (int64_t)a.group_base + (int64_t)tile_idx * Hkv + kvh;
    const int64_t slot0 = grp * a.max_splits;
    const int nsp = tile.n_splits;
    // buffer resources based at this group's partials; sc1 (cache-policy bit
    // 16) makes the accesses coherent across the XCDs' L2s
    constexpr int kCoherent = 16;
    const __amdgpu_buffer_rsrc_t racc = __builtin_amdgcn_make_buffer_rsrc(
        a.part_acc + slot0 * NP * kThreads * 4, 0, kRawRecords, kRawWord3);
    const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(
        a.part_ml + slot0 * kThreads * 2, 0, kRawRecords, kRawWord3);
    auto acc_off = [&](int sp, int j) __attribute__((always_inline)) { return ((sp * NP + j) * kThreads + tid) * 16; };
    auto ml_off = [&](int sp) __attribute__((always_inline)) { return (sp * kThreads + tid) * 8; };
    {
        // the column's total l adds the partner half-wave's
        const float l_col = pair_sum(l_run);
        const float inv = l_col > 0.0f ? 1.0f / l_col : 0.0f;
        uint64_t* pacc = reinterpret_cast<uint64_t*>(a.part_acc + slot0 * NP * kThreads * 4);
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const f32x16& x = acc[j >> 1];
            const int r0 = 8 * (j & 1);
            f16x8 h;
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (_Float16)(x[r0 + e] * inv);
            const u32x4 u = __builtin_bit_cast(u32x4, h);
            uint64_t* pp = pacc + acc_off(split, j) / 8;
            store_device2(pp, __uint_as_float(u[0]), __uint_as_float(u[1]));
            store_device2(pp + 1, __uint_as_float(u[2]), __uint_as_float(u[3]));
        }
        store_device2(reinterpret_cast<uint64_t*>(a.part_ml + slot0 * kThreads * 2) + ml_off(split) / 8,
                      m_run, l_col);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) sm.last = atomicAdd(a.counters + grp, 1) == nsp - 1;
    __syncthreads();
    if (!sm.last) return;
    if (tid == 0) __hip_atomic_store(a.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // Fold the splits in ascending order, two per round trip, this one's own
    // partial re-read like the others, so the result does not depend on which
    // split finishes last.  The running maximum M moves up as splits arrive
    // (acc and L rescaled then), so no separate pass over the splits' m is
    // needed; a column that no split saw (padding) keeps M = -inf: weights 0.
    float M = -INFINITY;
    float L = 0.0f;
    auto fold = [&](const u32x2& ml, const u32x4 (&x)[NP]) __attribute__((always_inline)) {
        const float m = __uint_as_float(ml[0]);
        if (m > M) {
            const float r = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - m);
            L *= r;
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] *= r;
            M = m;
        }
        const float w = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
        const float wl = w * __uint_as_float(ml[1]);
        L += wl;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const f16x8 h = __builtin_bit_cast(f16x8, x[j]);
            f32x16& t = acc[j >> 1];
            const int r0 = 8 * (j & 1);
#pragma unroll
            for (int e = 0; e < 8; ++e) t[r0 + e] = __builtin_fmaf(wl, (float)h[e], t[r0 + e]);
        }
    };
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.0f;
#pragma unroll 1
    for (int sp = 0; sp < nsp; sp += 2) {
        const int sp1 = min(sp + 1, nsp - 1);
        u32x4 x0[NP], x1[NP];
        const u32x2 ml0 = __builtin_amdgcn_raw_buffer_load_b64(rml, ml_off(sp), 0, kCoherent);
        const u32x2 ml1 = __builtin_amdgcn_raw_buffer_load_b64(rml, ml_off(sp1), 0, kCoherent);
#pragma unroll
        for (int j = 0; j < NP; ++j) x0[j] = __builtin_amdgcn_raw_buffer_load_b128(racc, acc_off(sp, j), 0, kCoherent);
#pragma unroll
        for (int j = 0; j < NP; ++j) x1[j] = __builtin_amdgcn_raw_buffer_load_b128(racc, acc_off(sp1, j), 0, kCoherent);
        fold(ml0, x0);
        if (sp + 1 < nsp) fold(ml1, x1);
    }
    // L is already the column's total (each split stored its column l)
    if (tok >= 0) write_out(L);
}

template <int D, bool ONE_PAGE, bool UNIFIED>
hipError_t launch_prefill_dpu(const PrefillArgs& a, const TileList& tl, int n_items, size_t lds,
                              hipStream_t stream) {
    const int G = a.n_q_heads / a.n_kv_heads;
    const dim3 grid((unsigned)n_items);
    const dim3 block(kThreads);
    switch (G) {
        case 1: hipLaunchKernelGGL((prefill_kernel<D, 1, ONE_PAGE, UNIFIED>), grid, block, lds, stream, a, tl); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<D, 2, ONE_PAGE, UNIFIED>), grid, block, lds, stream, a, tl); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<D, 4, ONE_PAGE, UNIFIED>), grid, block, lds, stream, a, tl); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<D, 8, ONE_PAGE, UNIFIED>), grid, block, lds, stream, a, tl); break;
        case 16: hipLaunchKernelGGL((prefill_kernel<D, 16, ONE_PAGE, UNIFIED>), grid, block, lds, stream, a, tl); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a, const TileList& tl, int n_items, size_t lds,
                            hipStream_t stream) {
    const bool one_page = a.page_size % kKvTile == 0;
    if (a.unified) {
        if (one_page) return launch_prefill_dpu<D, true, true>(a, tl, n_items, lds, stream);
        return launch_prefill_dpu<D, false, true>(a, tl, n_items, lds, stream);
    }
    if (one_page) return launch_prefill_dpu<D, true, false>(a, tl, n_items, lds, stream);
    return launch_prefill_dpu<D, false, false>(a, tl, n_items, lds, stream);
}

}  // namespace

int prefill_tokens_per_tile(int group) { return kRows / group; }

int prefill_threads() { return kThreads; }

int prefill_page_table_entries(int split_tokens, int page_size) {
    // a split starts at a multiple of the 64-key tile: its keys span at most
    // ceil(split_tokens / P) + 1 pages
    return (split_tokens + page_size - 1) / page_size + 1;
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillTile* tiles, int n_tiles,
                          hipStream_t stream) {
    if (n_tiles <= 0) return hipSuccess;
    if (n_tiles > kMaxTilesPerLaunch) return hipErrorInvalidValue;
    TileList tl;
    int items = 0;
    for (int i = 0; i < n_tiles; ++i) {
        tl.t[i] = tiles[i];
        tl.t[i].item0 = items;
        items += tiles[i].n_splits;
    }
    PrefillArgs b = a;
    b.n_tiles = n_tiles;
    const int n_items = items * a.n_kv_heads;
    const size_t lds = sizeof(int32_t) * (size_t)prefill_page_table_entries(a.split_tokens, a.page_size);
    if (a.head_dim == 128) return launch_prefill_d<128>(b, tl, n_items, lds, stream);
    return launch_prefill_d<64>(b, tl, n_items, lds, stream);
}


}  // namespace pa
