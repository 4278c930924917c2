/*
 * pa.h -- C ABI of libpa: paged attention over a block-table KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes is fixed by three pages:
 *   [UA]  "面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化",
 *         section 作品简介: the cache keeps a page mapping and a true KV length
 *         per sequence; for a ubatch, the page table and true length are
 *         expanded per query token in token order, and each query reads only
 *         the valid pages of its own sequence (UA-PagedAttention).
 *   [CF]  "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎", section 2
 *         (fixed-size blocks behind a block table; copy-on-write sharing of
 *         blocks) and section 3 (one-pass and partition-plus-reduce paged
 *         attention kernels; reshape-and-cache; block copy).
 *   [RS]  "面向边缘智能体推理的 llama.cpp KV Cache 共享与复用优化", section
 *         主要功能与技术路线: a shared prefix is read-only, each request's
 *         private suffix is allocated separately.
 *
 * Conventions used by every entry point
 *   - Every call returns pa_status (0 = PA_OK, negative = error).  On error,
 *     pa_last_error() returns a message for the calling thread.  No C++
 *     exception crosses this boundary.
 *   - Cache storage for one layer is two device arrays of IEEE binary16:
 *       K cache  [num_pages][n_kv_heads][page_size][head_dim]
 *       V cache  [num_pages][n_kv_heads][page_size / T][head_dim][T],
 *                T = min(page_size, 32)
 *     Cell (page p, slot s) of KV head h holds one token's key row
 *     K[p][h][s][:] and value column V[p][h][s / T][:][s % T]: a V page keeps
 *     its slots in blocks of T, each block slot-innermost (for page_size <= 32
 *     this is V[p][h][:][s]).  A slot id is page * page_size + slot.
 *   - Query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Device pointers are pa_dev pointers; the caller allocates and owns every
 *     device buffer.  Device calls are asynchronous on `stream` (a hipStream_t;
 *     NULL is the default stream) and only launch kernels: they do not
 *     allocate, copy host memory to the device, or synchronize.
 *   - Host pointers are read during the call only.
 *   - Supported shapes: head_dim in {64, 128}; page_size a power of two in
 *     [16, 1024]; n_q_heads a multiple of n_kv_heads with group size
 *     G = n_q_heads / n_kv_heads in {1, 2, 4, 8, 16}.  Other shapes return
 *     PA_ERR_UNSUPPORTED before anything is launched.
 *   - Block-table entries and slots are not range-checked on the device.
 *     pa_decode, pa_prefill and pa_reshape_and_cache take optional host
 *     copies of the tables they address through (block_tables_host,
 *     slot_mapping_host); when one is passed, every entry the launch would
 *     read is checked on the host first and a bad one returns PA_ERR_INVALID
 *     before anything is launched: page ids must lie in [0, num_pages), live
 *     slots in [0, num_pages*page_size) with none repeated.  Setting the
 *     environment variable PA_VALIDATE=1 (any value but "0") makes those host
 *     copies mandatory (PA_ERR_INVALID when one is NULL).  Without a host
 *     copy, an out-of-range page id or slot on the device is undefined
 *     behaviour.  Host copies must hold the same values as the device arrays.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID = -1,      /* bad argument or shape; nothing was changed or launched */
    PA_ERR_UNSUPPORTED = -2,  /* shape outside the supported set */
    PA_ERR_NO_PAGES = -3,     /* page pool exhausted; the pool is unchanged */
    PA_ERR_STATE = -4,        /* call not valid in the current pool state; pool unchanged */
    PA_ERR_HIP = -5,          /* the HIP runtime reported an error at launch */
    PA_ERR_WORKSPACE = -6     /* workspace missing or smaller than required */
} pa_status;

typedef void* pa_stream;      /* a hipStream_t */

/* Text describing the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/* Library version, as major*10000 + minor*100 + patch. */
int32_t pa_version(void);

/* ===================================================================== */
/* Host page pool and block tables ([CF] section 2; [UA] 作品简介; [RS]).  */
/* Host memory only; never touches the device.  Not thread-safe: one     */
/* thread at a time per pool.                                            */
/* ===================================================================== */

typedef struct pa_pool pa_pool;   /* opaque; created and freed by the library */

/* Create a pool of `num_pages` pages of `page_size` cells.  `free_order`
 * (nullable; else a permutation of 0..num_pages-1) is the order in which
 * free pages are handed out; NULL means 0, 1, 2, ...  The free list is a
 * stack: a page whose reference count falls to 0 is handed out next. */
pa_status pa_pool_create(int32_t num_pages, int32_t page_size, const int32_t* free_order,
                         pa_pool** out);
void      pa_pool_destroy(pa_pool* pool);

/* New empty sequence; its id is the smallest non-negative id not in use. */
pa_status pa_seq_new(pa_pool* pool, int32_t* seq_out);

/* Reserve cells for `n_new` more tokens of `seq`.  Fills the last page
 * before taking new pages.  Writes slot_mapping_out[i] = page*page_size +
 * slot for token i.  If the last page is shared (reference count > 1) and
 * partly filled, the sequence first gets a private copy of it: the pair
 * (source page, destination page) is written to cow_pair_out and *n_cow_out
 * is set to 1 (else 0).  The caller must run pa_copy_blocks on that pair
 * before writing the new tokens with pa_reshape_and_cache.  Fails with
 * PA_ERR_NO_PAGES, leaving the pool unchanged, if too few pages are free. */
pa_status pa_seq_append(pa_pool* pool, int32_t seq, int32_t n_new, int32_t* slot_mapping_out,
                        int32_t cow_pair_out[2], int32_t* n_cow_out);

/* New sequence sharing every page of `src` (reference counts + 1): the
 * read-only shared prefix of [RS]; later appends copy on write ([CF] §2). */
pa_status pa_seq_fork(pa_pool* pool, int32_t src_seq, int32_t* dst_seq_out);

/* Give `seq` a private copy of its logical page `logical_page`, which must be
 * shared (else PA_ERR_STATE).  Writes (source page, new page) to pair_out;
 * the caller copies it with pa_copy_blocks. */
pa_status pa_seq_cow(pa_pool* pool, int32_t seq, int32_t logical_page, int32_t pair_out[2]);

/* Release `seq`; its pages' reference counts drop by one and pages that reach
 * zero return to the free stack in logical order.  PA_ERR_STATE if `seq` is
 * not live. */
pa_status pa_seq_free(pa_pool* pool, int32_t seq);

/* Export the block tables and true lengths of `n` live sequences:
 * bt_out[i][j] = page of logical page j of seqs[i], -1 past its last page
 * (row-major [n][max_pages]); kv_len_out[i] = its number of tokens.
 * PA_ERR_INVALID if a sequence has more than max_pages pages. */
pa_status pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n, int32_t max_pages,
                          int32_t* bt_out, int32_t* kv_len_out);

/* Number of free pages, and (nullable) the reference count of every page
 * into refcount_out[num_pages]. */
pa_status pa_pool_stats(const pa_pool* pool, int32_t* n_free_out, int32_t* refcount_out);

/* Preemption and compaction ([CF] 内存管理策略 and 抢占与恢复机制: a preempted
 * sequence's blocks move to a reserved CPU area and come back without
 * recomputation; fragmented blocks are compacted into contiguous locations).
 *
 * pa_pool_host_reserve: the host reserve becomes n_host_pages page slots
 * (a stack, slot 0 handed out first).  PA_ERR_STATE while any sequence is
 * swapped out.
 *
 * pa_seq_swap_out: gives every page of a resident sequence, in logical order,
 * a host slot, writes the (device page, host slot) copies to make into
 * pairs_out[n][2] (*n_pairs_out = n, the sequence's page count) and drops the
 * sequence's device references (pages reaching 0 are pushed as by
 * pa_seq_free).  The caller copies with pa_swap_blocks(to_host = 1) before
 * those device pages are written again.  The sequence keeps its id; until
 * pa_seq_swap_in, only pa_seq_free accepts it (others: PA_ERR_STATE).
 * PA_ERR_NO_PAGES if the reserve has too few free slots, PA_ERR_INVALID if
 * max_pairs < n; failures change nothing.
 *
 * pa_seq_swap_in: takes a device page per host slot of a swapped-out
 * sequence, in logical order, writes the (host slot, device page) copies into
 * pairs_out (copy with pa_swap_blocks(to_host = 0) before reading the pages)
 * and returns the slots to the reserve.  The new pages are private
 * (refcount 1).  PA_ERR_NO_PAGES if too few device pages are free.
 *
 * pa_pool_compact: with n_live pages in use, moves every live page with id >=
 * n_live (ascending) onto the free ids below n_live (ascending), rewrites
 * every resident sequence's table, the prefix cache's pages (below) and the
 * refcounts, and leaves the free
 * stack n_live..N-1 with n_live handed out first.  The (src, dst) moves go to
 * pairs_out (at most num_pages); they satisfy pa_copy_blocks' rules, which
 * performs them on the device.
 *
 * pa_pool_host_stats: number of free host reserve slots. */
pa_status pa_pool_host_reserve(pa_pool* pool, int32_t n_host_pages);
pa_status pa_seq_swap_out(pa_pool* pool, int32_t seq, int32_t* pairs_out, int32_t max_pairs,
                          int32_t* n_pairs_out);
pa_status pa_seq_swap_in(pa_pool* pool, int32_t seq, int32_t* pairs_out, int32_t max_pairs,
                         int32_t* n_pairs_out);
pa_status pa_pool_compact(pa_pool* pool, int32_t* pairs_out, int32_t max_pairs, int32_t* n_pairs_out);
pa_status pa_pool_host_stats(const pa_pool* pool, int32_t* n_host_free_out);

/* Prefix cache: "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎", section
 * 核心架构与技术贡献 item 2 and section 前缀缓存优化 (a trie lookup reuses the KV
 * blocks of shared prefixes, such as a common system prompt), and
 * "面向边缘智能体推理的 llama.cpp KV Cache 共享与复用优化", section 主要功能与技术路线
 * (longest-prefix match over a token prefix tree, LRU reclaim of its leaves).
 * The tree's edges are whole pages of token ids (page_size int32 tokens), the
 * page being what two sequences can share without a copy; every cached node
 * holds one reference on its physical page.  Token ids are opaque int32.
 * Token arrays are host memory read during the call only.
 *
 * pa_prefix_insert: walks the first n_tokens / page_size full pages of
 * tokens (which must be the sequence's first tokens, n_tokens <= its length)
 * and caches each one not yet in the tree with the sequence's page at that
 * position (refcount + 1).  *n_cached_out (may be null) = cached pages on the
 * path.  Stamps the path as most recently used, then evicts over capacity.
 * PA_ERR_INVALID if a page to cache is already cached under another path (the
 * same sequence inserted with different tokens); failures change nothing.
 *
 * pa_prefix_match: follows full pages of tokens as far as the tree holds
 * them, stamps that path, and creates a new sequence (*seq_out) whose table is
 * those pages (refcount + 1 each) and whose length *n_matched_out is the
 * matched page count * page_size (0 if nothing matched).  The caller appends
 * the rest of its tokens to it; the length is page-aligned, so no shared page
 * is ever written.  The cache never pins a sequence: freeing it drops only
 * its own references.
 *
 * Eviction removes the leaf with the oldest stamp among leaves whose page no
 * sequence holds, so each removal frees exactly one page; a cached page that a
 * live or matched sequence still uses is not evicted.
 * pa_prefix_evict: frees up to n_pages pages this way (*n_freed_out).
 * pa_prefix_capacity: caps the cached page count (default num_pages) and
 * evicts down to it as far as eviction can; *n_freed_out may be null.
 * pa_prefix_stats: cached page count. */
pa_status pa_prefix_insert(pa_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                           int32_t* n_cached_out);
pa_status pa_prefix_match(pa_pool* pool, const int32_t* tokens, int32_t n_tokens, int32_t* seq_out,
                          int32_t* n_matched_out);
pa_status pa_prefix_evict(pa_pool* pool, int32_t n_pages, int32_t* n_freed_out);
pa_status pa_prefix_capacity(pa_pool* pool, int32_t max_pages, int32_t* n_freed_out);
pa_status pa_prefix_stats(const pa_pool* pool, int32_t* n_cached_out);

/* ===================================================================== */
/* Device operations.                                                    */
/* ===================================================================== */

typedef struct {
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv_heads;
    int32_t head_dim;
} pa_cache_desc;

/* Reshape-and-cache ([CF] section 3): write new tokens' keys and values into
 * their cells.  k_new, v_new: device [n_tokens][n_kv_heads][head_dim], binary16
 * (src_is_f32 = 0) or IEEE binary32 (src_is_f32 = 1, rounded to nearest even
 * on store).  slot_mapping: device int32 [n_tokens]; a negative slot skips the
 * token.  Live slots must be distinct and < num_pages*page_size.
 * slot_mapping_host: NULL or a host copy of slot_mapping, checked against those
 * rules before the launch (mandatory under PA_VALIDATE=1).  Bits are copied
 * exactly for binary16 input. */
pa_status pa_reshape_and_cache(const pa_cache_desc* desc, void* k_cache, void* v_cache,
                               const void* k_new, const void* v_new, int32_t src_is_f32,
                               const int32_t* slot_mapping, const int32_t* slot_mapping_host,
                               int32_t n_tokens, pa_stream stream);

/* Block copy for copy-on-write ([CF] sections 2 and 3): for every layer l and
 * pair i, copy page pairs_host[2i] onto page pairs_host[2i+1] in both
 * k_caches_host[l] and v_caches_host[l].  Pairs are validated on the host:
 * ids in range, no destination repeated, no destination that is also a
 * source (PA_ERR_INVALID otherwise).  k_caches_host / v_caches_host are host
 * arrays of n_layers device pointers.  Bits are copied exactly. */
pa_status pa_copy_blocks(const pa_cache_desc* desc, void* const* k_caches_host,
                         void* const* v_caches_host, int32_t n_layers, const int32_t* pairs_host,
                         int32_t n_pairs, pa_stream stream);

/* Block swap ([CF] section 3, the block copy/swap kernel; 抢占与恢复机制): for every
 * layer l and pair i, copy one whole page between the device pool
 * (k_caches_host[l], v_caches_host[l]: device pointers, layout of
 * pa_cache_desc) and a host reserve of n_host_pages pages of the same layout
 * (k_swap_host[l], v_swap_host[l]: pinned host memory mapped for the device,
 * e.g. from hipHostMalloc or torch's pin_memory).  to_host = 1: pairs are
 * (device page, host slot); 0: (host slot, device page).  Validated on the
 * host: ids in range, no destination repeated, host reserves pinned and mapped
 * (hipHostGetDevicePointer succeeds) -- PA_ERR_INVALID otherwise.  One kernel
 * launch per 128 pairs x 32 layers reads or writes the host pages directly;
 * bits are copied exactly. */
pa_status pa_swap_blocks(const pa_cache_desc* desc, void* const* k_caches_host,
                         void* const* v_caches_host, void* const* k_swap_host,
                         void* const* v_swap_host, int32_t n_host_pages, int32_t n_layers,
                         const int32_t* pairs_host, int32_t n_pairs, int32_t to_host,
                         pa_stream stream);

/* Workspace bytes pa_decode needs for these arguments (0 if it needs none).
 * Same meaning of arguments as pa_decode.  A decode workspace starts with
 * per-(sequence, KV head) completion counters (a region of
 * max(64 KiB, 4 * n_seqs * n_kv_heads) bytes) followed by split partials.
 * The counter region must be zero-filled before the workspace's first use;
 * every pa_decode call puts each counter it used back to zero before its
 * kernel ends, so the workspace can be reused by later calls on the same
 * stream, including calls of other shapes as long as
 * n_seqs * n_kv_heads <= 16384 (beyond that, re-zero it when the shape
 * changes).  Calls that overlap in time need different workspaces, and
 * nothing else may write to the workspace. */
size_t pa_decode_workspace_bytes(const pa_cache_desc* desc, int32_t n_seqs, int32_t n_q_heads,
                                 int32_t max_pages, const int32_t* kv_lens_host,
                                 int32_t partition_tokens);

/* Paged decode attention ([UA] 作品简介; [CF] section 3): one query token per
 * sequence at position kv_len-1, reading only the sequence's first kv_len
 * cells through its block-table row.  One kernel launch: when sequences are
 * split into partitions, the last workgroup of each (sequence, KV head)
 * combines them (log-sum-exp reduce).
 *   q            device fp32 [n_seqs][n_q_heads][head_dim]
 *   out          device fp32 [n_seqs][n_q_heads][head_dim]
 *   block_tables device int32 [n_seqs][max_pages]; only the first
 *                ceil(kv_len/page_size) entries of a row are read
 *   kv_lens      device int32 [n_seqs]; each in [1, max_pages*page_size]
 *   block_tables_host  host copy of block_tables or NULL; when given (it
 *                needs kv_lens_host), the entries each sequence reads are
 *                checked to be page ids in [0, num_pages) before the launch
 *   kv_lens_host host copy of kv_lens or NULL; sizes the split and bounds the
 *                table check (both host copies are mandatory under
 *                PA_VALIDATE=1)
 *   scale        softmax scale (e.g. 1/sqrt(head_dim))
 *   partition_tokens  0 = choose (about one workgroup per compute unit
 *                when all lengths are equal, partitions of at most 2048
 *                tokens otherwise; needs kv_lens_host); -1 = one pass per
 *                sequence (no split); >0 = split every sequence into
 *                partitions of this many tokens (a multiple of 256),
 *                combined by a log-sum-exp reduce.
 * The result does not depend on the physical page ids, and cells past a
 * sequence's length are never used, whatever they hold. */
pa_status pa_decode(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                    const float* q, float* out, const int32_t* block_tables,
                    const int32_t* kv_lens, const int32_t* block_tables_host,
                    const int32_t* kv_lens_host, int32_t n_seqs,
                    int32_t max_pages, int32_t n_q_heads, float scale, int32_t partition_tokens,
                    void* workspace, size_t workspace_bytes, pa_stream stream);

/* Paged decode that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, meaning, results and errors as
 * pa_decode, without the workspace: the split partials and completion
 * counters live in a fixed device array of the library (one per GPU, of
 * pa_decode_noalloc_scratch_bytes() = 32 MiB, held until the process ends).
 * The caller still passes every input and output.  Limits, checked before any
 * launch: pa_decode_workspace_bytes() for the same arguments must not exceed
 * the scratch size (else PA_ERR_WORKSPACE), and n_seqs * n_kv_heads must not
 * exceed 16384 (else PA_ERR_UNSUPPORTED).  No call allocates: the first call
 * on a device looks the array up and clears its counters with one small kernel
 * on `stream`.  Every call on a GPU uses that GPU's one array, so calls that
 * overlap in time on one GPU (other streams, other threads) race; calls on
 * one stream may follow one another in any shapes. */
pa_status pa_decode_noalloc(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                            const float* q, float* out, const int32_t* block_tables,
                            const int32_t* kv_lens, const int32_t* block_tables_host,
                            const int32_t* kv_lens_host, int32_t n_seqs, int32_t max_pages,
                            int32_t n_q_heads, float scale, int32_t partition_tokens,
                            pa_stream stream);
size_t    pa_decode_noalloc_scratch_bytes(void);

/* Workspace bytes pa_prefill needs for these arguments (0 if no tile's KV
 * range is split).  Same meaning of arguments as pa_prefill.  A prefill
 * workspace starts with per-(tile, KV head) completion counters (a region of
 * max(64 KiB, 4 * tiles * n_kv_heads) bytes, tiles <= n_tokens) followed by
 * split partials; the counter region follows the same rules as pa_decode's:
 * zero-filled before first use, left zeroed by every call, reusable across
 * calls (and with pa_decode) on one stream while the region stays within
 * 64 KiB, one workspace per concurrently running call. */
size_t pa_prefill_workspace_bytes(const pa_cache_desc* desc, int32_t n_tokens, int32_t n_q_heads,
                                  const int32_t* token_row_host, const int32_t* token_kv_len_host,
                                  const int32_t* token_pos_host, int32_t kv_splits);

/* UA paged prefill ([UA] 作品简介): attention for one ubatch whose tokens may
 * come from several sequences in any order.  One kernel launch per 128 tiles
 * (plus one that zeroes padding rows if there are any): when a tile's KV
 * range is split, the last split to finish combines the partials.  Token i carries its sequence's
 * block-table row token_row[i] (-1 = padding token: its output row is set to
 * 0), the sequence's true KV length token_kv_len[i] (K/V of this ubatch
 * already written) and its position token_pos[i]; it attends to cells
 * t < min(token_kv_len[i], token_pos[i] + 1) of that row.
 *   q            device fp32 [n_tokens][n_q_heads][head_dim]; rounded to
 *                binary16 (nearest even) for the matrix products, which
 *                accumulate in fp32; a split KV range's partial output
 *                (normalised by its own row sum) is rounded to binary16
 *                before the splits are combined in fp32
 *   out          device fp32 [n_tokens][n_q_heads][head_dim]
 *   block_tables device int32 [n_rows][max_pages]
 *   token_row, token_kv_len, token_pos   device int32 [n_tokens]
 *   token_row_host, token_kv_len_host, token_pos_host   host copies of the
 *                same arrays, used to plan the work (grouping tokens by
 *                sequence); they must equal the device arrays
 *   block_tables_host  host copy of block_tables or NULL; when given, the
 *                entries every row's tokens read (up to the row's longest
 *                visible range) are checked to be page ids in
 *                [0, num_pages) before the launch (mandatory under
 *                PA_VALIDATE=1)
 *   kv_splits    0 = choose (splits widened until the launch has about one
 *                workgroup per compute unit: right when this launch has
 *                the GPU to itself); >= 1 = split each tile's KV range into
 *                at most this many parts combined by a log-sum-exp reduce.
 *                1 (no split, no partials, no combine) suits callers that
 *                keep several launches in flight on separate streams, whose
 *                workgroups then fill the GPU together
 * Each row's tokens are grouped into tiles in ubatch order; a tile's work
 * ends at its last token's visible length, so tokens of a row should appear
 * in increasing position for efficiency (not for correctness). */
pa_status pa_prefill(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                     const float* q, float* out, const int32_t* block_tables,
                     const int32_t* token_row, const int32_t* token_kv_len,
                     const int32_t* token_pos, const int32_t* token_row_host,
                     const int32_t* token_kv_len_host, const int32_t* token_pos_host,
                     const int32_t* block_tables_host, int32_t n_tokens, int32_t n_rows,
                     int32_t max_pages, int32_t n_q_heads, float scale, int32_t kv_splits,
                     void* workspace, size_t workspace_bytes, pa_stream stream);

/* ---------------------------------------------------------------------------
 * Unified-span attention: the baseline UA-PagedAttention replaces ([UA]
 * 作品简介): with several sequences in one unified KV cache, every query of a
 * ubatch faces one physical span of cells from all sequences, free cells and
 * padding; the mask removes the cells that do not belong to the query from
 * the result but not from the data access and the computation.  Provided to
 * measure the paged path against it on the same pool.
 *
 * The span is cells 0..span-1 of the pool read as one flat array: cell c is
 * page c / page_size, slot c % page_size.  Every token scans all span cells.
 *   q, out       device fp32 [n_tokens][n_q_heads][head_dim] (q rounded to
 *                binary16 for the products, as in pa_prefill)
 *   cell_seq     device int32 [span]: sequence id whose position cell_pos[c]
 *                cell c holds, -1 for a free or padding cell (its K and V may
 *                hold anything, NaN included)
 *   cell_pos     device int32 [span]
 *   token_seq    device int32 [n_tokens]: the token's sequence (-1 = padding)
 *   token_pos    device int32 [n_tokens]: the token's position
 * Token i attends to the cells with cell_seq == token_seq[i] and cell_pos <=
 * token_pos[i]; a padding token, or one that sees no cell, gets a zero row.
 * Limits: sequence ids in [0, 512) and positions in [0, 2^22) (cells and
 * tokens); outside them the mask is undefined (no out-of-bounds access).
 * span must be in [1, num_pages * page_size] (PA_ERR_INVALID otherwise).
 * kv_splits and the workspace follow pa_prefill's rules (same counter
 * contract). */
size_t pa_unified_workspace_bytes(const pa_cache_desc* desc, int32_t n_tokens, int32_t n_q_heads,
                                  int32_t span, int32_t kv_splits);
pa_status pa_unified_attention(const pa_cache_desc* desc, const void* k_cache, const void* v_cache,
                               const float* q, float* out, int32_t span, const int32_t* cell_seq,
                               const int32_t* cell_pos, const int32_t* token_seq,
                               const int32_t* token_pos, int32_t n_tokens, int32_t n_q_heads,
                               float scale, int32_t kv_splits, void* workspace,
                               size_t workspace_bytes, pa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
