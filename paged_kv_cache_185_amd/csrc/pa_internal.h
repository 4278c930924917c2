// Internal declarations shared by the C-ABI layer (api.cpp) and the kernel
// translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "pa.h"

namespace pa {

// Message for pa_last_error() on the calling thread.
void set_error(const std::string& msg);

// pa_decode's validation, planning and launch with a given workspace.
pa_status run_decode(const pa_cache_desc* desc, const void* k_cache, const void* v_cache, const float* q,
                     float* out, const int32_t* block_tables, const int32_t* kv_lens,
                     const int32_t* block_tables_host, const int32_t* kv_lens_host, int32_t n_seqs,
                     int32_t max_pages, int32_t n_q_heads, float scale, int32_t partition_tokens,
                     void* workspace, size_t workspace_bytes, pa_stream stream);

// ---- V page layout ----------------------------------------------------------
// A V page of one KV head holds its slots in blocks of T = min(P, kVSlotTile)
// consecutive slots, each block a [head_dim][T] array (slot innermost), blocks
// in slot order.  Every 32-token run that a decode chunk or half a prefill
// tile reads is then one contiguous 8 KiB block (D = 128), where a [D][P] page
// would give it 64-byte pieces on a 2P-byte stride.  For P <= 32 this is the
// [D][P] page.
constexpr int kVSlotTile = 32;

__host__ __device__ inline int v_slot_tile(int page_size) {
    return page_size < kVSlotTile ? page_size : kVSlotTile;
}

// element offset of V(page, KV head h, value dim d, slot) in a V cache
__host__ __device__ inline int64_t v_elem_offset(int64_t page, int h, int d, int slot, int n_kv_heads,
                                                 int page_size, int head_dim) {
    const int T = v_slot_tile(page_size);
    return ((page * n_kv_heads + h) * page_size + (slot & ~(T - 1))) * head_dim + (int64_t)d * T +
           (slot & (T - 1));
}

// ---- reshape_and_cache / copy_blocks -------------------------------------

hipError_t launch_reshape_and_cache(void* k_cache, void* v_cache, const void* k_new,
                                    const void* v_new, bool src_f32, const int32_t* slots,
                                    int32_t n_tokens, int32_t n_kv_heads, int32_t page_size,
                                    int32_t head_dim, hipStream_t stream);

// Copies up to kMaxCopyPairs pairs for up to kMaxCopyLayers layers per launch.
constexpr int kMaxCopyPairs = 128;
constexpr int kMaxCopyLayers = 32;
// Page copies from src to dst page arrays of one layout (pairs: src page, dst page).
hipError_t launch_copy_pages(void* const* src_k, void* const* dst_k, void* const* src_v,
                             void* const* dst_v, int32_t n_layers, const int32_t* pairs, int32_t n_pairs,
                             int64_t page_bytes, hipStream_t stream);
hipError_t launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t n_layers,
                              const int32_t* pairs, int32_t n_pairs, int64_t page_bytes,
                              hipStream_t stream);

// ---- decode ---------------------------------------------------------------

// Tokens per partition are a multiple of this (the tokens one round of the
// decode workgroup's 8 waves streams: 8 x 32-token chunks).
constexpr int kDecodePartitionQuantum = 256;

struct DecodeArgs {
    const uint16_t* k_cache;
    const uint16_t* v_cache;
    const float* q;
    float* out;
    const int32_t* block_tables;
    const int32_t* kv_lens;
    float* part_m;      // [n_seqs][Hq][n_part] (log2 domain), or null for one pass
    float* part_l;      // [n_seqs][Hq][n_part]
    float* part_acc;    // [n_seqs][Hq][n_part][D]
    int32_t* counters;  // [n_seqs][Hkv] finished partitions; zero between calls
    int32_t n_seqs;
    int32_t max_pages;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t page_size;  // a power of two
    int32_t page_shift; // log2(page_size)
    int32_t head_dim;
    int32_t partition_tokens;
    int32_t n_part;     // partitions per sequence in the grid
    float scale_log2;   // scale * log2(e)
};

// Batches of up to kDecodeItemSeqs sequences launch only their live
// (sequence, partition) items: item0[s] is the first item of sequence s
// (items numbered sequence by sequence); n_seqs = 0 launches every
// (partition, sequence) pair and lets the empty ones exit.
constexpr int kDecodeItemSeqs = 1024;
struct DecodeItems {
    int32_t n_seqs;
    int32_t item0[kDecodeItemSeqs + 1];
};

hipError_t launch_decode(const DecodeArgs& a, const DecodeItems& items, int64_t n_workgroups,
                         hipStream_t stream);
// LDS entries the decode kernel needs for one partition's page ids.
int decode_page_table_entries(int partition_tokens, int page_size);
// Largest page-id table the decode kernel stages in LDS (32 KiB).
constexpr int kDecodeMaxPageEntries = 8192;
// Largest automatic decode partition when the batch's lengths differ.
constexpr int64_t kDecodeVarlenPartition = 2048;
// Minimum size of the completion-counter region at the start of a decode
// workspace (16384 counters).
constexpr size_t kDecodeCounterBytes = 65536;


// ---- prefill ---------------------------------------------------------------

// One tile = the tokens of one sequence (block-table row) that a workgroup
// handles for one KV head.  Tokens are found on the device by scanning
// token_row[first .. last] for `row`; exactly `count` of them match.
struct PrefillTile {
    int32_t row;
    int32_t first;      // ubatch index of the tile's first token
    int32_t last;       // ubatch index of the tile's last token
    int32_t count;      // tokens in the tile (<= tokens per tile)
    int32_t kv_end;     // largest visible length of any token in the tile
    int32_t min_vis;    // smallest visible length of any token in the tile
    int32_t n_splits;   // KV splits used by this tile (<= grid splits)
    int32_t dense;      // 1: the tile's tokens are first, first+1, ..., last
    int32_t item0;      // first (tile, split) item of the tile in its launch (set at launch)
    int32_t split_len;  // keys per split of this tile (multiple of the KV tile)
};

constexpr int kMaxTilesPerLaunch = 128;

struct PrefillArgs {
    const uint16_t* k_cache;
    const uint16_t* v_cache;
    const float* q;
    float* out;
    const int32_t* block_tables;
    const int32_t* token_row;
    const int32_t* token_kv_len;
    const int32_t* token_pos;
    // split partials (null when no tile splits), slot = group*max_splits+split
    // with group = tile*Hkv + kvh over all tiles of the call:
    int32_t* counters;  // [groups], zero between calls
    float* part_ml;     // [slot][threads][2]  (m, the column l)
    float* part_acc;    // [slot][D/16][threads] 16-byte pieces of binary16 o = acc / l, lane order
    int32_t n_tokens;
    int32_t max_pages;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t page_size;  // a power of two
    int32_t page_shift; // log2(page_size)
    int32_t head_dim;
    int32_t split_tokens;   // the longest split of any tile (sizes the LDS page table)
    int32_t max_splits;     // split slots per (token, head) in the partials
    int32_t n_tiles;        // tiles in the current launch (set by launch_prefill)
    int32_t group_base;     // first group of the current launch
    float scale_log2;
    // unified-span mode (pa_unified_attention): keys are cells 0..span-1 of the
    // pool read as one flat array; cell c holds position cell_pos[c] of
    // sequence cell_seq[c] (-1 = free); token_row holds each token's sequence
    int32_t unified;
    const int32_t* cell_seq;
    const int32_t* cell_pos;
};

int prefill_tokens_per_tile(int group);   // query tokens per tile for GQA group size
int prefill_threads();                    // threads per prefill workgroup
constexpr int kPrefillKvTile = 64;
// LDS entries the prefill kernel needs for one split's page ids, and the cap.
int prefill_page_table_entries(int split_tokens, int page_size);
constexpr int kPrefillMaxPageEntries = 8192;

hipError_t launch_prefill(const PrefillArgs& a, const PrefillTile* tiles, int n_tiles,
                          hipStream_t stream);

// Zero the output rows of padding tokens (token_row < 0).
hipError_t launch_zero_rows(float* out, const int32_t* token_row, int32_t n_tokens,
                            int32_t row_elems, hipStream_t stream);

}  // namespace pa
