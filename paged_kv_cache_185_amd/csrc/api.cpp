// C-ABI entry points for the device operations: argument validation, work
// planning (partition sizes for decode, token tiles and KV splits for
// prefill) and kernel launches on the caller's stream.  No device memory is
// allocated here and nothing is copied from the host to the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace pa {

static thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }

namespace {

constexpr double kLog2e = 1.4426950408889634;

pa_status fail(pa_status st, const std::string& msg) {
    set_error(msg);
    return st;
}

pa_status hip_fail(const char* where, hipError_t e) {
    return fail(PA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool validate_env() {
    const char* v = std::getenv("PA_VALIDATE");
    return v && v[0] && v[0] != '0';
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

int32_t log2_exact(int32_t x) {
    int32_t s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

pa_status check_desc(const char* fn, const pa_cache_desc* d) {
    if (!d) return fail(PA_ERR_INVALID, std::string(fn) + ": desc is null");
    if (d->num_pages < 1 || d->n_kv_heads < 1 || d->page_size < 1 || d->head_dim < 1)
        return fail(PA_ERR_INVALID, std::string(fn) + ": cache dimensions must be >= 1");
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(PA_ERR_UNSUPPORTED, std::string(fn) + ": head_dim must be 64 or 128");
    if (d->page_size < 16 || d->page_size > 1024 || (d->page_size & (d->page_size - 1)) != 0)
        return fail(PA_ERR_UNSUPPORTED,
                    std::string(fn) + ": page_size must be a power of two in [16, 1024]");
    if ((int64_t)d->num_pages * d->page_size > INT32_MAX)
        return fail(PA_ERR_INVALID, std::string(fn) + ": num_pages * page_size overflows int32 slots");
    return PA_OK;
}

pa_status check_heads(const char* fn, const pa_cache_desc* d, int32_t n_q_heads) {
    if (n_q_heads < 1 || n_q_heads % d->n_kv_heads != 0)
        return fail(PA_ERR_INVALID, std::string(fn) + ": n_q_heads must be a multiple of n_kv_heads");
    const int G = n_q_heads / d->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
        return fail(PA_ERR_UNSUPPORTED, std::string(fn) + ": GQA group size must be 1, 2, 4, 8 or 16");
    return PA_OK;
}

// ---------------------------------------------------------- host range checks
//
// Block-table entries and slots are used as addresses on the device without a
// check there.  When the caller passes host copies, the entries a launch would
// read are checked here first; PA_VALIDATE=1 makes the host copies mandatory.

// Entries [0, ceil(n_cells / P)) of `row` must be page ids in [0, num_pages).
pa_status check_table_row(const char* fn, const pa_cache_desc* d, const int32_t* bt_host, int32_t max_pages,
                          int64_t row, int64_t n_cells) {
    const int64_t n = (n_cells + d->page_size - 1) / d->page_size;
    if (n > max_pages)
        return fail(PA_ERR_INVALID, std::string(fn) + ": row " + std::to_string(row) +
                                        " needs more than max_pages entries");
    const int32_t* r = bt_host + row * (int64_t)max_pages;
    for (int64_t j = 0; j < n; ++j)
        if (r[j] < 0 || r[j] >= d->num_pages)
            return fail(PA_ERR_INVALID, std::string(fn) + ": block_tables[" + std::to_string(row) + "][" +
                                            std::to_string(j) + "] = " + std::to_string(r[j]) +
                                            " is not a page id in [0, num_pages)");
    return PA_OK;
}

// ---------------------------------------------------------------- decode plan

struct DecodePlan {
    int32_t partition_tokens = 0;
    int32_t n_part = 1;
    size_t cnt_off = 0, m_off = 0, l_off = 0, acc_off = 0, bytes = 0;
};

pa_status plan_decode(const pa_cache_desc* d, int32_t n_seqs, int32_t n_q_heads, int32_t max_pages,
                      const int32_t* kv_lens_host, int32_t partition_tokens, DecodePlan* plan) {
    if (n_seqs < 0 || max_pages < 1)
        return fail(PA_ERR_INVALID, "pa_decode: n_seqs must be >= 0 and max_pages >= 1");
    const int64_t cap = (int64_t)max_pages * d->page_size;
    int64_t total = (int64_t)n_seqs * cap, longest = cap;
    int64_t shortest = longest;
    if (kv_lens_host) {
        total = 0;
        longest = 1;
        shortest = INT64_MAX;
        for (int32_t i = 0; i < n_seqs; ++i) {
            const int64_t L = kv_lens_host[i];
            if (L < 1 || L > cap)
                return fail(PA_ERR_INVALID, "pa_decode: kv_len must be in [1, max_pages*page_size]");
            total += L;
            longest = std::max(longest, L);
            shortest = std::min(shortest, L);
        }
    }
    const int64_t Q = kDecodePartitionQuantum;
    int64_t T;
    if (partition_tokens == -1) {
        T = round_up(longest, Q);
    } else if (partition_tokens > 0) {
        if (partition_tokens % Q != 0)
            return fail(PA_ERR_INVALID, "pa_decode: partition_tokens must be a multiple of 256");
        T = partition_tokens;
    } else if (partition_tokens == 0) {
        // about one workgroup (8 waves streaming one partition) per compute
        // unit: measured faster on the 256-CU part than more, shorter
        // partitions, and it keeps the split partials small
        const int64_t work = total * d->n_kv_heads;
        T = std::max<int64_t>(Q, round_up((work + 255) / 256, Q));
        // with unequal lengths the workgroups differ in size and the largest
        // ones end last: partitions of at most kDecodeVarlenPartition tokens
        // let the dispatcher even the load out (measured on mixed batches of
        // 256..32768 tokens with the live-only grid: 2048-token partitions
        // 3-4% faster than 4096, and a third faster than one partition per
        // compute unit's share)
        if (shortest != longest) T = std::min<int64_t>(T, kDecodeVarlenPartition);
        if (T >= longest) T = round_up(longest, Q);
    } else {
        return fail(PA_ERR_INVALID, "pa_decode: partition_tokens must be -1, 0 or a positive multiple of 256");
    }
    // the kernel stages one partition's page ids in LDS: cap the partition so
    // the table fits (a "one pass" request beyond that becomes a split)
    const int64_t t_cap = (int64_t)(kDecodeMaxPageEntries - 1) * d->page_size / Q * Q;
    T = std::min(T, t_cap);
    plan->partition_tokens = (int32_t)std::min<int64_t>(T, INT32_MAX / 2);
    plan->n_part = (int32_t)((longest + T - 1) / T);
    // one workgroup per (partition, KV head, sequence) in a one-dimensional grid
    if ((int64_t)plan->n_part * d->n_kv_heads * n_seqs > INT32_MAX)
        return fail(PA_ERR_INVALID, "pa_decode: partitions x KV heads x sequences exceeds the grid limit");
    if (plan->n_part > 1) {
        const size_t rows = (size_t)n_seqs * n_q_heads * plan->n_part;
        // completion counters first, in a region of at least 64 KiB, so the
        // partials of a call with n_seqs * n_kv_heads <= 16384 never land on
        // another call's counters when one workspace serves several shapes
        plan->cnt_off = 0;
        plan->m_off = align256(std::max<size_t>(kDecodeCounterBytes, (size_t)n_seqs * d->n_kv_heads * 4));
        plan->l_off = plan->m_off + align256(rows * 4);
        plan->acc_off = plan->l_off + align256(rows * 4);
        plan->bytes = plan->acc_off + align256(rows * (size_t)d->head_dim * 4);
    }
    return PA_OK;
}

// --------------------------------------------------------------- prefill plan

struct PrefillPlan {
    std::vector<PrefillTile> tiles;
    int32_t split_tokens = 0;
    int32_t max_splits = 1;
    bool has_padding = false;
    size_t ml_off = 0, acc_off = 0, bytes = 0;
};

// Per-tile KV split lengths and counts and the workspace layout, given the tiles.
pa_status finish_prefill_plan(const pa_cache_desc* d, int32_t kv_splits, int64_t max_kv,
                              PrefillPlan* plan) {
    const int64_t KT = kPrefillKvTile;
    // the kernel stages one split's page ids in LDS: very long ranges are split
    const int64_t lds_cap = (int64_t)(kPrefillMaxPageEntries - 1) * d->page_size / KT * KT;
    auto kv_of = [](const PrefillTile& t) { return std::max<int64_t>(t.kv_end, 1); };
    if (kv_splits >= 1) {
        // the same split length for every tile
        int64_t split = kv_splits == 1 ? round_up(std::max<int64_t>(max_kv, 1), KT)
                                       : round_up(std::max<int64_t>((max_kv + kv_splits - 1) / kv_splits, 1), KT);
        split = std::min(split, lds_cap);
        for (auto& t : plan->tiles) {
            t.split_len = (int32_t)split;
            t.n_splits = (int32_t)((kv_of(t) + split - 1) / split);
        }
    } else {
        // one 8-wave workgroup fits a compute unit (256 CUs): at most
        // 256 / Hkv (tile, split) pairs per KV head keep the grid to one
        // round of workgroups (the excess of a larger grid runs as a second
        // round).  The pairs go one at a time to the tile whose splits are
        // longest, splits no shorter than 256 keys; each tile's range is
        // then cut into equal splits, so no tile carries a short remainder
        // split beside full ones.
        const int64_t need = std::max<int64_t>(1, 256 / d->n_kv_heads);
        const size_t n = plan->tiles.size();
        std::vector<int64_t> cnt(n);
        int64_t pairs = 0;
        for (size_t i = 0; i < n; ++i) {
            cnt[i] = (kv_of(plan->tiles[i]) + lds_cap - 1) / lds_cap;
            pairs += cnt[i];
        }
        auto len = [&](size_t i, int64_t c) { return (kv_of(plan->tiles[i]) + c - 1) / c; };
        while (pairs < need) {
            size_t best = n;
            for (size_t i = 0; i < n; ++i)
                if (best == n || len(i, cnt[i]) > len(best, cnt[best])) best = i;
            if (best == n || len(best, cnt[best] + 1) < 256) break;
            ++cnt[best];
            ++pairs;
        }
        for (size_t i = 0; i < n; ++i) {
            auto& t = plan->tiles[i];
            const int64_t split = std::min(lds_cap, round_up(len(i, cnt[i]), KT));
            t.split_len = (int32_t)split;
            t.n_splits = (int32_t)((kv_of(t) + split - 1) / split);
        }
    }
    plan->split_tokens = 0;
    plan->max_splits = 1;
    for (const auto& t : plan->tiles) {
        plan->split_tokens = std::max(plan->split_tokens, t.split_len);
        plan->max_splits = std::max(plan->max_splits, t.n_splits);
    }
    if (plan->max_splits > 1) {
        // counters first (zero-filled region shared with pa_decode's
        // convention), then per (tile, KV head, split) slot the (m, l) pairs
        // and the binary16 normalised outputs of every lane of the workgroup
        const size_t groups = plan->tiles.size() * (size_t)d->n_kv_heads;
        const size_t slots = groups * plan->max_splits;
        const size_t threads = (size_t)prefill_threads();
        plan->ml_off = align256(std::max<size_t>(kDecodeCounterBytes, groups * 4));
        plan->acc_off = plan->ml_off + align256(slots * threads * 2 * 4);
        // per lane: head_dim/2 outputs in binary16 (head_dim bytes)
        plan->bytes = plan->acc_off + align256(slots * threads * (size_t)d->head_dim);
    }
    return PA_OK;
}

pa_status plan_prefill(const pa_cache_desc* d, int32_t n_tokens, int32_t n_q_heads, int32_t n_rows,
                       int32_t max_pages, const int32_t* row, const int32_t* kv_len,
                       const int32_t* pos, int32_t kv_splits, PrefillPlan* plan) {
    if (n_tokens < 0) return fail(PA_ERR_INVALID, "pa_prefill: n_tokens < 0");
    if (n_tokens > 0 && (!row || !kv_len || !pos))
        return fail(PA_ERR_INVALID, "pa_prefill: host token arrays are required");
    if (kv_splits < 0) return fail(PA_ERR_INVALID, "pa_prefill: kv_splits < 0");
    const int G = n_q_heads / d->n_kv_heads;
    const int tpt = prefill_tokens_per_tile(G);
    const int64_t cap = max_pages > 0 ? (int64_t)max_pages * d->page_size : INT64_MAX;
    std::vector<int32_t> order;
    order.reserve(n_tokens);
    for (int32_t i = 0; i < n_tokens; ++i) {
        if (row[i] < 0) {
            plan->has_padding = true;
            continue;
        }
        if (n_rows >= 0 && row[i] >= n_rows)
            return fail(PA_ERR_INVALID, "pa_prefill: token_row out of range");
        if (pos[i] < 0 || kv_len[i] < 1 || (int64_t)kv_len[i] > cap)
            return fail(PA_ERR_INVALID, "pa_prefill: need pos >= 0 and kv_len in [1, max_pages*page_size]");
        order.push_back(i);
    }
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t x, int32_t y) { return row[x] < row[y]; });
    int64_t max_kv = 0;
    for (size_t b = 0; b < order.size();) {
        size_t e = b;
        while (e < order.size() && row[order[e]] == row[order[b]]) ++e;
        for (size_t s = b; s < e; s += tpt) {
            const size_t f = std::min(e, s + tpt);
            PrefillTile t{};
            t.row = row[order[s]];
            t.first = order[s];
            t.last = order[f - 1];
            t.count = (int32_t)(f - s);
            int32_t ke = 0, kmin = INT32_MAX;
            for (size_t j = s; j < f; ++j) {
                const int32_t i = order[j];
                const int32_t vis = std::min(kv_len[i], pos[i] + 1);
                ke = std::max(ke, vis);
                kmin = std::min(kmin, vis);
            }
            t.kv_end = ke;
            t.min_vis = kmin;
            t.dense = (t.last - t.first + 1 == t.count) ? 1 : 0;
            plan->tiles.push_back(t);
            max_kv = std::max<int64_t>(max_kv, ke);
        }
        b = e;
    }
    return finish_prefill_plan(d, kv_splits, max_kv, plan);
}

// Unified span: tiles are runs of consecutive ubatch tokens, each scanning all
// `span` cells.
pa_status plan_unified(const pa_cache_desc* d, int32_t n_tokens, int32_t n_q_heads, int32_t span,
                       int32_t kv_splits, PrefillPlan* plan) {
    if (n_tokens < 0) return fail(PA_ERR_INVALID, "pa_unified_attention: n_tokens < 0");
    if (kv_splits < 0) return fail(PA_ERR_INVALID, "pa_unified_attention: kv_splits < 0");
    if (span < 1 || (int64_t)span > (int64_t)d->num_pages * d->page_size)
        return fail(PA_ERR_INVALID, "pa_unified_attention: span must be in [1, num_pages*page_size]");
    const int tpt = prefill_tokens_per_tile(n_q_heads / d->n_kv_heads);
    for (int32_t b = 0; b < n_tokens; b += tpt) {
        PrefillTile t{};
        t.row = 0;
        t.first = b;
        t.last = std::min(n_tokens, b + tpt) - 1;
        t.count = t.last - t.first + 1;
        t.kv_end = span;
        t.min_vis = 0;
        t.dense = 1;
        plan->tiles.push_back(t);
    }
    return finish_prefill_plan(d, kv_splits, span, plan);
}

// Fill the common launch arguments from a plan and launch its tiles (at most
// kMaxTilesPerLaunch per launch) on `stream`.
pa_status run_prefill_plan(const char* who, const pa_cache_desc* desc, const PrefillPlan& plan,
                           PrefillArgs a, const void* k_cache, const void* v_cache, const float* q,
                           float* out, int32_t n_tokens, int32_t n_q_heads, float scale,
                           void* workspace, pa_stream stream) {
    a.k_cache = (const uint16_t*)k_cache;
    a.v_cache = (const uint16_t*)v_cache;
    a.q = q;
    a.out = out;
    if (plan.max_splits > 1) {
        char* ws = (char*)workspace;
        a.counters = (int32_t*)ws;
        a.part_ml = (float*)(ws + plan.ml_off);
        a.part_acc = (float*)(ws + plan.acc_off);
    }
    a.n_tokens = n_tokens;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = desc->n_kv_heads;
    a.page_size = desc->page_size;
    a.page_shift = log2_exact(desc->page_size);
    a.head_dim = desc->head_dim;
    a.split_tokens = plan.split_tokens;
    a.max_splits = plan.max_splits;
    a.scale_log2 = (float)((double)scale * kLog2e);
    const int n_tiles = (int)plan.tiles.size();
    for (int b = 0; b < n_tiles; b += kMaxTilesPerLaunch) {
        const int nb = std::min(kMaxTilesPerLaunch, n_tiles - b);
        a.group_base = b * desc->n_kv_heads;
        hipError_t e = launch_prefill(a, plan.tiles.data() + b, nb, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(who, e);
    }
    return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_last_error(void) { return g_error.c_str(); }

int32_t pa_version(void) { return 200; }

pa_status pa_reshape_and_cache(const pa_cache_desc* desc, void* k_cache, void* v_cache,
                               const void* k_new, const void* v_new, int32_t src_is_f32,
                               const int32_t* slot_mapping, const int32_t* slot_mapping_host,
                               int32_t n_tokens, pa_stream stream) {
    pa_status st = check_desc("pa_reshape_and_cache", desc);
    if (st != PA_OK) return st;
    if (n_tokens < 0) return fail(PA_ERR_INVALID, "pa_reshape_and_cache: n_tokens < 0");
    if (n_tokens == 0) return PA_OK;
    if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
        return fail(PA_ERR_INVALID, "pa_reshape_and_cache: null pointer");
    if (src_is_f32 != 0 && src_is_f32 != 1)
        return fail(PA_ERR_INVALID, "pa_reshape_and_cache: src_is_f32 must be 0 or 1");
    if (validate_env() && !slot_mapping_host)
        return fail(PA_ERR_INVALID, "pa_reshape_and_cache: PA_VALIDATE=1 needs slot_mapping_host");
    if (slot_mapping_host) {
        // live slots inside the pool, none written twice (the result would
        // depend on which write lands last)
        const int64_t n_slots = (int64_t)desc->num_pages * desc->page_size;
        std::vector<int32_t> live;
        live.reserve(n_tokens);
        for (int32_t i = 0; i < n_tokens; ++i) {
            const int32_t sl = slot_mapping_host[i];
            if (sl < 0) continue;
            if (sl >= n_slots)
                return fail(PA_ERR_INVALID, "pa_reshape_and_cache: slot_mapping[" + std::to_string(i) + "] = " +
                                                std::to_string(sl) + " is past the pool");
            live.push_back(sl);
        }
        std::sort(live.begin(), live.end());
        if (std::adjacent_find(live.begin(), live.end()) != live.end())
            return fail(PA_ERR_INVALID, "pa_reshape_and_cache: a slot is written twice");
    }
    hipError_t e = launch_reshape_and_cache(k_cache, v_cache, k_new, v_new, src_is_f32 == 1,
                                            slot_mapping, n_tokens, desc->n_kv_heads,
                                            desc->page_size, desc->head_dim, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : hip_fail("pa_reshape_and_cache", e);
}

pa_status pa_copy_blocks(const pa_cache_desc* desc, void* const* k_caches_host,
                         void* const* v_caches_host, int32_t n_layers, const int32_t* pairs_host,
                         int32_t n_pairs, pa_stream stream) {
    pa_status st = check_desc("pa_copy_blocks", desc);
    if (st != PA_OK) return st;
    if (n_layers < 0 || n_pairs < 0) return fail(PA_ERR_INVALID, "pa_copy_blocks: negative count");
    if (n_layers == 0 || n_pairs == 0) return PA_OK;
    if (!k_caches_host || !v_caches_host || !pairs_host)
        return fail(PA_ERR_INVALID, "pa_copy_blocks: null pointer");
    for (int32_t l = 0; l < n_layers; ++l)
        if (!k_caches_host[l] || !v_caches_host[l])
            return fail(PA_ERR_INVALID, "pa_copy_blocks: null cache pointer");
    std::vector<char> is_dst(desc->num_pages, 0), is_src(desc->num_pages, 0);
    for (int32_t i = 0; i < n_pairs; ++i) {
        const int32_t s = pairs_host[2 * i], dpg = pairs_host[2 * i + 1];
        if (s < 0 || s >= desc->num_pages || dpg < 0 || dpg >= desc->num_pages)
            return fail(PA_ERR_INVALID, "pa_copy_blocks: page id out of range");
        if (is_dst[dpg]) return fail(PA_ERR_INVALID, "pa_copy_blocks: a destination repeats");
        is_dst[dpg] = 1;
        is_src[s] = 1;
    }
    for (int32_t p = 0; p < desc->num_pages; ++p)
        if (is_dst[p] && is_src[p])
            return fail(PA_ERR_INVALID, "pa_copy_blocks: a destination is also a source");
    const int64_t page_bytes =
        (int64_t)desc->n_kv_heads * desc->page_size * desc->head_dim * 2;
    hipError_t e = launch_copy_blocks(k_caches_host, v_caches_host, n_layers, pairs_host, n_pairs,
                                      page_bytes, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : hip_fail("pa_copy_blocks", e);
}

pa_status pa_swap_blocks(const pa_cache_desc* desc, void* const* k_caches_host,
                         void* const* v_caches_host, void* const* k_swap_host,
                         void* const* v_swap_host, int32_t n_host_pages, int32_t n_layers,
                         const int32_t* pairs_host, int32_t n_pairs, int32_t to_host,
                         pa_stream stream) {
    pa_status st = check_desc("pa_swap_blocks", desc);
    if (st != PA_OK) return st;
    if (n_layers < 0 || n_pairs < 0 || n_host_pages < 0)
        return fail(PA_ERR_INVALID, "pa_swap_blocks: negative count");
    if (to_host != 0 && to_host != 1) return fail(PA_ERR_INVALID, "pa_swap_blocks: to_host must be 0 or 1");
    if (n_layers == 0 || n_pairs == 0) return PA_OK;
    if (!k_caches_host || !v_caches_host || !k_swap_host || !v_swap_host || !pairs_host)
        return fail(PA_ERR_INVALID, "pa_swap_blocks: null pointer");
    for (int32_t l = 0; l < n_layers; ++l)
        if (!k_caches_host[l] || !v_caches_host[l] || !k_swap_host[l] || !v_swap_host[l])
            return fail(PA_ERR_INVALID, "pa_swap_blocks: null cache pointer");
    const int32_t n_src = to_host ? desc->num_pages : n_host_pages;
    const int32_t n_dst = to_host ? n_host_pages : desc->num_pages;
    std::vector<char> is_dst(n_dst, 0);
    for (int32_t i = 0; i < n_pairs; ++i) {
        const int32_t s = pairs_host[2 * i], dpg = pairs_host[2 * i + 1];
        if (s < 0 || s >= n_src || dpg < 0 || dpg >= n_dst)
            return fail(PA_ERR_INVALID, "pa_swap_blocks: page or slot id out of range");
        if (is_dst[dpg]) return fail(PA_ERR_INVALID, "pa_swap_blocks: a destination repeats");
        is_dst[dpg] = 1;
    }
    const int64_t page_bytes =
        (int64_t)desc->n_kv_heads * desc->page_size * desc->head_dim * 2;
    // the kernel reaches the host reserve through its device mapping; memory
    // that is not pinned and mapped is rejected here, never dereferenced
    std::vector<void*> kh(n_layers), vh(n_layers);
    for (int32_t l = 0; l < n_layers; ++l) {
        if (hipHostGetDevicePointer(&kh[l], k_swap_host[l], 0) != hipSuccess ||
            hipHostGetDevicePointer(&vh[l], v_swap_host[l], 0) != hipSuccess) {
            (void)hipGetLastError();
            return fail(PA_ERR_INVALID, "pa_swap_blocks: host reserve is not pinned, mapped memory");
        }
    }
    hipError_t e = to_host ? launch_copy_pages(k_caches_host, kh.data(), v_caches_host, vh.data(),
                                               n_layers, pairs_host, n_pairs, page_bytes, (hipStream_t)stream)
                           : launch_copy_pages(kh.data(), k_caches_host, vh.data(), v_caches_host,
                                               n_layers, pairs_host, n_pairs, page_bytes, (hipStream_t)stream);
    return e == hipSuccess ? PA_OK : hip_fail("pa_swap_blocks", e);
}

size_t pa_decode_workspace_bytes(const pa_cache_desc* desc, int32_t n_seqs, int32_t n_q_heads,
                                 int32_t max_pages, const int32_t* kv_lens_host,
                                 int32_t partition_tokens) {
    if (check_desc("pa_decode_workspace_bytes", desc) != PA_OK) return 0;
    if (check_heads("pa_decode_workspace_bytes", desc, n_q_heads) != PA_OK) return 0;
    DecodePlan plan;
    if (plan_decode(desc, n_seqs, n_q_heads, max_pages, kv_lens_host, partition_tokens, &plan) != PA_OK)
        return 0;
    return plan.bytes;
}

pa_status pa_decode(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                    const float* q, float* out, const int32_t* block_tables,
                    const int32_t* kv_lens, const int32_t* block_tables_host,
                    const int32_t* kv_lens_host, int32_t n_seqs,
                    int32_t max_pages, int32_t n_q_heads, float scale, int32_t partition_tokens,
                    void* workspace, size_t workspace_bytes, pa_stream stream) {
    return pa::run_decode(desc, k_cache, v_cache, q, out, block_tables, kv_lens, block_tables_host,
                          kv_lens_host, n_seqs, max_pages, n_q_heads, scale, partition_tokens, workspace,
                          workspace_bytes, stream);
}

}  // extern "C"

// Validation, planning and the launch of pa_decode, given the workspace (also
// the path of pa_decode_noalloc, whose workspace is the library's scratch).
pa_status pa::run_decode(const pa_cache_desc* desc, const void* k_cache, const void* v_cache, const float* q,
                         float* out, const int32_t* block_tables, const int32_t* kv_lens,
                         const int32_t* block_tables_host, const int32_t* kv_lens_host, int32_t n_seqs,
                         int32_t max_pages, int32_t n_q_heads, float scale, int32_t partition_tokens,
                         void* workspace, size_t workspace_bytes, pa_stream stream) {
    pa_status st = check_desc("pa_decode", desc);
    if (st != PA_OK) return st;
    if ((st = check_heads("pa_decode", desc, n_q_heads)) != PA_OK) return st;
    if (n_seqs == 0) return PA_OK;
    if (!k_cache || !v_cache || !q || !out || !block_tables || !kv_lens)
        return fail(PA_ERR_INVALID, "pa_decode: null pointer");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "pa_decode: scale must be finite");
    DecodePlan plan;
    if ((st = plan_decode(desc, n_seqs, n_q_heads, max_pages, kv_lens_host, partition_tokens, &plan)) != PA_OK)
        return st;
    if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes))
        return fail(PA_ERR_WORKSPACE, "pa_decode: workspace missing or too small (need " +
                                          std::to_string(plan.bytes) + " bytes)");
    if (validate_env() && (kv_lens_host == nullptr || block_tables_host == nullptr))
        return fail(PA_ERR_INVALID, "pa_decode: PA_VALIDATE=1 needs kv_lens_host and block_tables_host");
    if (block_tables_host) {
        if (!kv_lens_host)
            return fail(PA_ERR_INVALID, "pa_decode: checking block_tables_host needs kv_lens_host");
        for (int32_t i = 0; i < n_seqs; ++i)
            if ((st = check_table_row("pa_decode", desc, block_tables_host, max_pages, i, kv_lens_host[i])) != PA_OK)
                return st;
    }
    DecodeArgs a{};
    a.k_cache = (const uint16_t*)k_cache;
    a.v_cache = (const uint16_t*)v_cache;
    a.q = q;
    a.out = out;
    a.block_tables = block_tables;
    a.kv_lens = kv_lens;
    if (plan.n_part > 1) {
        char* ws = (char*)workspace;
        a.counters = (int32_t*)(ws + plan.cnt_off);
        a.part_m = (float*)(ws + plan.m_off);
        a.part_l = (float*)(ws + plan.l_off);
        a.part_acc = (float*)(ws + plan.acc_off);
    }
    a.n_seqs = n_seqs;
    a.max_pages = max_pages;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = desc->n_kv_heads;
    a.page_size = desc->page_size;
    a.page_shift = log2_exact(desc->page_size);
    a.head_dim = desc->head_dim;
    a.partition_tokens = plan.partition_tokens;
    a.n_part = plan.n_part;
    a.scale_log2 = (float)((double)scale * kLog2e);
    // live (sequence, partition) items only, when the lengths are known here
    // and the table fits the kernel argument
    static thread_local DecodeItems items;
    int64_t n_workgroups = (int64_t)plan.n_part * desc->n_kv_heads * n_seqs;
    items.n_seqs = 0;
    if (kv_lens_host && n_seqs > 0 && n_seqs <= kDecodeItemSeqs) {
        int64_t total = 0;
        for (int32_t i = 0; i < n_seqs; ++i) {
            items.item0[i] = (int32_t)total;
            total += ((int64_t)kv_lens_host[i] + plan.partition_tokens - 1) / plan.partition_tokens;
        }
        items.item0[n_seqs] = (int32_t)total;
        items.n_seqs = n_seqs;
        n_workgroups = total * desc->n_kv_heads;
    }
    if (n_workgroups == 0) return PA_OK;
    hipError_t e = launch_decode(a, items, n_workgroups, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("pa_decode", e);
    return PA_OK;
}

extern "C" {

size_t pa_prefill_workspace_bytes(const pa_cache_desc* desc, int32_t n_tokens, int32_t n_q_heads,
                                  const int32_t* token_row_host, const int32_t* token_kv_len_host,
                                  const int32_t* token_pos_host, int32_t kv_splits) {
    if (check_desc("pa_prefill_workspace_bytes", desc) != PA_OK) return 0;
    if (check_heads("pa_prefill_workspace_bytes", desc, n_q_heads) != PA_OK) return 0;
    PrefillPlan plan;
    if (plan_prefill(desc, n_tokens, n_q_heads, -1, -1, token_row_host, token_kv_len_host,
                     token_pos_host, kv_splits, &plan) != PA_OK)
        return 0;
    return plan.bytes;
}

pa_status pa_prefill(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                     const float* q, float* out, const int32_t* block_tables,
                     const int32_t* token_row, const int32_t* token_kv_len,
                     const int32_t* token_pos, const int32_t* token_row_host,
                     const int32_t* token_kv_len_host, const int32_t* token_pos_host,
                     const int32_t* block_tables_host, int32_t n_tokens, int32_t n_rows,
                     int32_t max_pages, int32_t n_q_heads, float scale, int32_t kv_splits,
                     void* workspace, size_t workspace_bytes, pa_stream stream) {
    pa_status st = check_desc("pa_prefill", desc);
    if (st != PA_OK) return st;
    if ((st = check_heads("pa_prefill", desc, n_q_heads)) != PA_OK) return st;
    if (n_tokens == 0) return PA_OK;
    if (!k_cache || !v_cache || !q || !out || !block_tables || !token_row || !token_kv_len ||
        !token_pos)
        return fail(PA_ERR_INVALID, "pa_prefill: null pointer");
    if (n_rows < 1 || max_pages < 1)
        return fail(PA_ERR_INVALID, "pa_prefill: n_rows and max_pages must be >= 1");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "pa_prefill: scale must be finite");
    PrefillPlan plan;
    if ((st = plan_prefill(desc, n_tokens, n_q_heads, n_rows, max_pages, token_row_host,
                           token_kv_len_host, token_pos_host, kv_splits, &plan)) != PA_OK)
        return st;
    if (validate_env() && !block_tables_host)
        return fail(PA_ERR_INVALID, "pa_prefill: PA_VALIDATE=1 needs block_tables_host");
    if (block_tables_host) {
        // the entries a tile reads: those of its row up to the longest visible
        // range of its tokens
        std::vector<int64_t> vis(n_rows, 0);
        for (int32_t i = 0; i < n_tokens; ++i) {
            const int32_t r = token_row_host[i];
            if (r >= 0) vis[r] = std::max<int64_t>(vis[r], std::min(token_kv_len_host[i], token_pos_host[i] + 1));
        }
        for (int32_t r = 0; r < n_rows; ++r)
            if (vis[r] > 0 &&
                (st = check_table_row("pa_prefill", desc, block_tables_host, max_pages, r, vis[r])) != PA_OK)
                return st;
    }
    if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes))
        return fail(PA_ERR_WORKSPACE, "pa_prefill: workspace missing or too small (need " +
                                          std::to_string(plan.bytes) + " bytes)");
    PrefillArgs a{};
    a.block_tables = block_tables;
    a.token_row = token_row;
    a.token_kv_len = token_kv_len;
    a.token_pos = token_pos;
    a.max_pages = max_pages;
    if ((st = run_prefill_plan("pa_prefill", desc, plan, a, k_cache, v_cache, q, out, n_tokens,
                               n_q_heads, scale, workspace, stream)) != PA_OK)
        return st;
    if (plan.has_padding) {
        hipError_t e = launch_zero_rows(out, token_row, n_tokens, n_q_heads * desc->head_dim,
                                        (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail("pa_prefill (padding rows)", e);
    }
    return PA_OK;
}

size_t pa_unified_workspace_bytes(const pa_cache_desc* desc, int32_t n_tokens, int32_t n_q_heads,
                                  int32_t span, int32_t kv_splits) {
    if (check_desc("pa_unified_workspace_bytes", desc) != PA_OK) return 0;
    if (check_heads("pa_unified_workspace_bytes", desc, n_q_heads) != PA_OK) return 0;
    PrefillPlan plan;
    if (plan_unified(desc, n_tokens, n_q_heads, span, kv_splits, &plan) != PA_OK) return 0;
    return plan.bytes;
}

pa_status pa_unified_attention(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                               const float* q, float* out, int32_t span, const int32_t* cell_seq,
                               const int32_t* cell_pos, const int32_t* token_seq,
                               const int32_t* token_pos, int32_t n_tokens, int32_t n_q_heads,
                               float scale, int32_t kv_splits, void* workspace,
                               size_t workspace_bytes, pa_stream stream) {
    pa_status st = check_desc("pa_unified_attention", desc);
    if (st != PA_OK) return st;
    if ((st = check_heads("pa_unified_attention", desc, n_q_heads)) != PA_OK) return st;
    if (n_tokens == 0) return PA_OK;
    if (!k_cache || !v_cache || !q || !out || !cell_seq || !cell_pos || !token_seq || !token_pos)
        return fail(PA_ERR_INVALID, "pa_unified_attention: null pointer");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "pa_unified_attention: scale must be finite");
    PrefillPlan plan;
    if ((st = plan_unified(desc, n_tokens, n_q_heads, span, kv_splits, &plan)) != PA_OK) return st;
    if (plan.bytes > 0 && (!workspace || workspace_bytes < plan.bytes))
        return fail(PA_ERR_WORKSPACE, "pa_unified_attention: workspace missing or too small (need " +
                                          std::to_string(plan.bytes) + " bytes)");
    PrefillArgs a{};
    a.token_row = token_seq;
    a.token_pos = token_pos;
    a.unified = 1;
    a.cell_seq = cell_seq;
    a.cell_pos = cell_pos;
    return run_prefill_plan("pa_unified_attention", desc, plan, a, k_cache, v_cache, q, out,
                            n_tokens, n_q_heads, scale, workspace, stream);
}

}  // extern "C"
