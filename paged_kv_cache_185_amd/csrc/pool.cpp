// Host page pool and block tables.
//
// Structure from "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎", section 2
// (fixed-size blocks mapped by a block table, copy-on-write sharing), and from
// "面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化", section 作品简介
// (a page mapping and a true length per sequence).  Sharing semantics from
// "面向边缘智能体推理的 llama.cpp KV Cache 共享与复用优化", section 主要功能与技术路线
// (read-only shared prefix, private suffix per request, budget over the union
// of physical cells -- here: a page is counted once, whatever its refcount).
//
// Policy (fixes the choice the pages leave open, so block tables are unique):
// a stack of free pages seeded so that free_order[0] is handed out first; freed
// pages are pushed in logical order; ids are the smallest unused; every call
// checks all its preconditions before changing anything.
//
// Preemption and compaction ("CacheFlow", sections 内存管理策略 and 抢占与恢复机制:
// blocks of a preempted sequence go to a reserved CPU area and return without
// recomputation; fragmented blocks are compacted into contiguous locations):
// the host reserve is a second stack of page slots (slot 0 on top); swap-out
// and swap-in walk the sequence's pages in logical order; compaction moves the
// live pages with ids >= n_live (ascending) onto the free ids below n_live
// (ascending) and leaves the free stack n_live..N-1 with n_live on top.
//
// Prefix cache ("CacheFlow", section 核心架构与技术贡献 item 2 and section 前缀缓存优化:
// a trie lookup reuses the blocks of shared prefixes; "面向边缘智能体推理的 llama.cpp
// KV Cache 共享与复用优化", section 主要功能与技术路线: longest-prefix match and LRU
// reclaim of leaves).  The tree's edges are whole pages of token ids, a page being
// the unit two sequences can share without a copy; each node holds one reference
// on its page.  Every insert and match stamps the nodes on its root path with a
// clock that then advances, so a parent's stamp is never below its children's
// and no two leaves share a stamp.  Eviction removes the least recently stamped
// leaf whose page nobody else holds, so each removal frees one page.
#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa.h"

namespace pa {
void set_error(const std::string& msg);
}

struct pa_pool {
    int32_t num_pages = 0;
    int32_t page_size = 0;
    std::vector<int32_t> free_stack;   // back() is the top
    std::vector<int32_t> ref;
    std::vector<int32_t> host_free;    // host reserve slots, back() is the top
    int32_t n_host = 0;
    int32_t n_swapped = 0;
    struct Seq {
        bool live = false;      // id in use
        bool swapped = false;   // pages are in the host reserve
        int64_t len = 0;
        std::vector<int32_t> pages;   // device pages, or host slots while swapped
    };
    std::vector<Seq> seqs;

    // prefix tree; node 0 is the root and holds no page
    struct Node {
        int32_t parent = -1;
        int32_t page = -1;
        int32_t n_children = 0;
        uint64_t stamp = 0;
        std::string key;   // parent id then the page's tokens, as raw bytes
    };
    std::vector<Node> nodes{Node{}};
    std::vector<int32_t> free_nodes;
    std::unordered_map<std::string, int32_t> child;   // Node::key -> node
    std::map<uint64_t, int32_t> leaves;               // stamp -> leaf node
    std::vector<int32_t> node_of_page;                // page -> node, or -1
    int32_t n_cached = 0;
    int32_t capacity = 0;
    uint64_t clock = 0;

    std::string edge(int32_t parent, const int32_t* toks) const {
        std::string k(sizeof(int32_t) * (1 + (size_t)page_size), '\0');
        std::memcpy(&k[0], &parent, sizeof(int32_t));
        std::memcpy(&k[sizeof(int32_t)], toks, sizeof(int32_t) * (size_t)page_size);
        return k;
    }
    int32_t find_child(int32_t parent, const int32_t* toks) const {
        auto it = child.find(edge(parent, toks));
        return it == child.end() ? -1 : it->second;
    }
    void restamp(int32_t n, uint64_t c) {
        Node& x = nodes[n];
        if (x.n_children == 0) leaves.erase(x.stamp);
        x.stamp = c;
        if (x.n_children == 0) leaves[c] = n;
    }
    int32_t add_node(int32_t parent, const int32_t* toks, int32_t page, uint64_t c) {
        int32_t n;
        if (!free_nodes.empty()) {
            n = free_nodes.back();
            free_nodes.pop_back();
        } else {
            nodes.emplace_back();
            n = (int32_t)nodes.size() - 1;
        }
        Node& x = nodes[n];
        x.parent = parent;
        x.page = page;
        x.n_children = 0;
        x.stamp = c;
        x.key = edge(parent, toks);
        child[x.key] = n;
        // the parent stops being a leaf before the child, which may carry the
        // same stamp, enters the leaf set
        if (parent != 0 && nodes[parent].n_children == 0) leaves.erase(nodes[parent].stamp);
        nodes[parent].n_children++;
        leaves[c] = n;
        node_of_page[page] = n;
        ref[page] += 1;
        n_cached += 1;
        return n;
    }
    // Frees cached pages in LRU order while more() holds; returns how many.
    // Leaves below the cursor were found held by someone else; removing one
    // leaf changes no other page's count, and a parent that becomes a leaf has
    // a stamp at least the cursor's, so the scan never has to go back.
    template <class More>
    int32_t evict(More more) {
        int32_t freed = 0;
        uint64_t cur = 0;
        while (more()) {
            auto it = leaves.lower_bound(cur);
            while (it != leaves.end() && ref[nodes[it->second].page] != 1) ++it;
            if (it == leaves.end()) break;
            cur = it->first;
            const int32_t n = it->second;
            leaves.erase(it);
            Node& x = nodes[n];
            child.erase(x.key);
            node_of_page[x.page] = -1;
            ref[x.page] = 0;
            free_stack.push_back(x.page);
            const int32_t parent = x.parent;
            x = Node{};
            free_nodes.push_back(n);
            n_cached -= 1;
            if (--nodes[parent].n_children == 0 && parent != 0) leaves[nodes[parent].stamp] = parent;
            freed += 1;
        }
        return freed;
    }
    int32_t evict_over_capacity() {
        return evict([this] { return n_cached > capacity; });
    }

    int32_t pop() {
        int32_t p = free_stack.back();
        free_stack.pop_back();
        return p;
    }
    bool in_use(int32_t s) const {
        return s >= 0 && s < (int32_t)seqs.size() && seqs[s].live;
    }
    // live and resident on the device
    bool live(int32_t s) const { return in_use(s) && !seqs[s].swapped; }
    int32_t new_id() {
        for (size_t i = 0; i < seqs.size(); ++i)
            if (!seqs[i].live) return (int32_t)i;
        seqs.emplace_back();
        return (int32_t)seqs.size() - 1;
    }
};

static pa_status fail(pa_status st, const char* msg) {
    pa::set_error(msg);
    return st;
}

extern "C" {

pa_status pa_pool_create(int32_t num_pages, int32_t page_size, const int32_t* free_order,
                         pa_pool** out) {
    if (!out) return fail(PA_ERR_INVALID, "pa_pool_create: out is null");
    *out = nullptr;
    if (num_pages < 1 || page_size < 1)
        return fail(PA_ERR_INVALID, "pa_pool_create: num_pages and page_size must be >= 1");
    if ((int64_t)num_pages * page_size > INT32_MAX)
        return fail(PA_ERR_INVALID, "pa_pool_create: num_pages * page_size overflows int32 slots");
    std::vector<int32_t> order(num_pages);
    if (free_order) {
        std::vector<char> seen(num_pages, 0);
        for (int32_t i = 0; i < num_pages; ++i) {
            int32_t p = free_order[i];
            if (p < 0 || p >= num_pages || seen[p])
                return fail(PA_ERR_INVALID, "pa_pool_create: free_order is not a permutation");
            seen[p] = 1;
            order[i] = p;
        }
    } else {
        for (int32_t i = 0; i < num_pages; ++i) order[i] = i;
    }
    pa_pool* pool = new (std::nothrow) pa_pool();
    if (!pool) return fail(PA_ERR_INVALID, "pa_pool_create: out of host memory");
    pool->num_pages = num_pages;
    pool->page_size = page_size;
    pool->free_stack.assign(order.rbegin(), order.rend());
    pool->ref.assign(num_pages, 0);
    pool->node_of_page.assign(num_pages, -1);
    pool->capacity = num_pages;
    *out = pool;
    return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

pa_status pa_seq_new(pa_pool* pool, int32_t* seq_out) {
    if (!pool || !seq_out) return fail(PA_ERR_INVALID, "pa_seq_new: null argument");
    int32_t id = pool->new_id();
    pool->seqs[id].live = true;
    pool->seqs[id].swapped = false;
    pool->seqs[id].len = 0;
    pool->seqs[id].pages.clear();
    *seq_out = id;
    return PA_OK;
}

pa_status pa_seq_append(pa_pool* pool, int32_t seq, int32_t n_new, int32_t* slot_mapping_out,
                        int32_t cow_pair_out[2], int32_t* n_cow_out) {
    if (!pool) return fail(PA_ERR_INVALID, "pa_seq_append: pool is null");
    if (!pool->live(seq)) return fail(PA_ERR_STATE, "pa_seq_append: sequence is not live");
    if (n_new < 0) return fail(PA_ERR_INVALID, "pa_seq_append: n_new < 0");
    if (n_new > 0 && !slot_mapping_out)
        return fail(PA_ERR_INVALID, "pa_seq_append: slot_mapping_out is null");
    auto& s = pool->seqs[seq];
    const int64_t P = pool->page_size;
    const int64_t L = s.len;
    if (n_cow_out) *n_cow_out = 0;
    if (n_new == 0) return PA_OK;
    const bool cow = (L % P) != 0 && pool->ref[s.pages.back()] > 1;
    const int64_t need = (L + n_new + P - 1) / P - (L + P - 1) / P + (cow ? 1 : 0);
    if (need > (int64_t)pool->free_stack.size())
        return fail(PA_ERR_NO_PAGES, "pa_seq_append: page pool exhausted");
    if (cow && (!cow_pair_out || !n_cow_out))
        return fail(PA_ERR_INVALID, "pa_seq_append: copy-on-write needed but cow outputs are null");
    if (cow) {
        int32_t src = s.pages.back();
        int32_t dst = pool->pop();
        pool->ref[src] -= 1;
        pool->ref[dst] = 1;
        s.pages.back() = dst;
        cow_pair_out[0] = src;
        cow_pair_out[1] = dst;
        *n_cow_out = 1;
    }
    for (int32_t j = 0; j < n_new; ++j) {
        int64_t t = L + j;
        if (t % P == 0) {
            int32_t p = pool->pop();
            pool->ref[p] = 1;
            s.pages.push_back(p);
        }
        slot_mapping_out[j] = (int32_t)(s.pages[t / P] * P + t % P);
    }
    s.len = L + n_new;
    return PA_OK;
}

pa_status pa_seq_fork(pa_pool* pool, int32_t src_seq, int32_t* dst_seq_out) {
    if (!pool || !dst_seq_out) return fail(PA_ERR_INVALID, "pa_seq_fork: null argument");
    if (!pool->live(src_seq)) return fail(PA_ERR_STATE, "pa_seq_fork: source is not live");
    int32_t id = pool->new_id();               // may grow seqs: take copies after
    auto& d = pool->seqs[id];
    const auto& s = pool->seqs[src_seq];
    d.live = true;
    d.swapped = false;
    d.len = s.len;
    d.pages = s.pages;
    for (int32_t p : d.pages) pool->ref[p] += 1;
    *dst_seq_out = id;
    return PA_OK;
}

pa_status pa_seq_cow(pa_pool* pool, int32_t seq, int32_t logical_page, int32_t pair_out[2]) {
    if (!pool || !pair_out) return fail(PA_ERR_INVALID, "pa_seq_cow: null argument");
    if (!pool->live(seq)) return fail(PA_ERR_STATE, "pa_seq_cow: sequence is not live");
    auto& s = pool->seqs[seq];
    if (logical_page < 0 || logical_page >= (int32_t)s.pages.size())
        return fail(PA_ERR_INVALID, "pa_seq_cow: logical page out of range");
    int32_t src = s.pages[logical_page];
    if (pool->ref[src] < 2) return fail(PA_ERR_STATE, "pa_seq_cow: page is not shared");
    if (pool->free_stack.empty()) return fail(PA_ERR_NO_PAGES, "pa_seq_cow: page pool exhausted");
    int32_t dst = pool->pop();
    pool->ref[src] -= 1;
    pool->ref[dst] = 1;
    s.pages[logical_page] = dst;
    pair_out[0] = src;
    pair_out[1] = dst;
    return PA_OK;
}

pa_status pa_seq_free(pa_pool* pool, int32_t seq) {
    if (!pool) return fail(PA_ERR_INVALID, "pa_seq_free: pool is null");
    if (!pool->in_use(seq)) return fail(PA_ERR_STATE, "pa_seq_free: sequence is not live");
    auto& s = pool->seqs[seq];
    if (s.swapped) {
        for (int32_t h : s.pages) pool->host_free.push_back(h);
        pool->n_swapped -= 1;
    } else {
        for (int32_t p : s.pages) {
            if (--pool->ref[p] == 0) pool->free_stack.push_back(p);
        }
    }
    s.swapped = false;
    s.pages.clear();
    s.len = 0;
    s.live = false;
    return PA_OK;
}

pa_status pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n, int32_t max_pages,
                          int32_t* bt_out, int32_t* kv_len_out) {
    if (!pool || (n > 0 && (!seqs || !bt_out || !kv_len_out)) || n < 0 || max_pages < 0)
        return fail(PA_ERR_INVALID, "pa_block_tables: bad argument");
    for (int32_t i = 0; i < n; ++i) {
        if (!pool->live(seqs[i])) return fail(PA_ERR_STATE, "pa_block_tables: sequence is not live");
        if ((int32_t)pool->seqs[seqs[i]].pages.size() > max_pages)
            return fail(PA_ERR_INVALID, "pa_block_tables: max_pages too small");
        if (pool->seqs[seqs[i]].len > INT32_MAX)
            return fail(PA_ERR_INVALID, "pa_block_tables: length overflows int32");
    }
    for (int32_t i = 0; i < n; ++i) {
        const auto& s = pool->seqs[seqs[i]];
        int32_t* row = bt_out + (int64_t)i * max_pages;
        for (int32_t j = 0; j < max_pages; ++j)
            row[j] = j < (int32_t)s.pages.size() ? s.pages[j] : -1;
        kv_len_out[i] = (int32_t)s.len;
    }
    return PA_OK;
}

pa_status pa_pool_stats(const pa_pool* pool, int32_t* n_free_out, int32_t* refcount_out) {
    if (!pool || !n_free_out) return fail(PA_ERR_INVALID, "pa_pool_stats: null argument");
    *n_free_out = (int32_t)pool->free_stack.size();
    if (refcount_out) std::copy(pool->ref.begin(), pool->ref.end(), refcount_out);
    return PA_OK;
}

pa_status pa_pool_host_reserve(pa_pool* pool, int32_t n_host_pages) {
    if (!pool || n_host_pages < 0) return fail(PA_ERR_INVALID, "pa_pool_host_reserve: bad argument");
    if (pool->n_swapped > 0)
        return fail(PA_ERR_STATE, "pa_pool_host_reserve: sequences are swapped out");
    pool->n_host = n_host_pages;
    pool->host_free.resize(n_host_pages);
    for (int32_t i = 0; i < n_host_pages; ++i) pool->host_free[i] = n_host_pages - 1 - i;
    return PA_OK;
}

pa_status pa_seq_swap_out(pa_pool* pool, int32_t seq, int32_t* pairs_out, int32_t max_pairs,
                          int32_t* n_pairs_out) {
    if (!pool || !n_pairs_out) return fail(PA_ERR_INVALID, "pa_seq_swap_out: null argument");
    if (!pool->live(seq)) return fail(PA_ERR_STATE, "pa_seq_swap_out: sequence is not resident");
    auto& s = pool->seqs[seq];
    const int32_t n = (int32_t)s.pages.size();
    if (n > max_pairs || (n > 0 && !pairs_out))
        return fail(PA_ERR_INVALID, "pa_seq_swap_out: pairs_out too small");
    if (n > (int32_t)pool->host_free.size())
        return fail(PA_ERR_NO_PAGES, "pa_seq_swap_out: host reserve exhausted");
    std::vector<int32_t> slots(n);
    for (int32_t j = 0; j < n; ++j) {
        slots[j] = pool->host_free.back();
        pool->host_free.pop_back();
        pairs_out[2 * j] = s.pages[j];
        pairs_out[2 * j + 1] = slots[j];
    }
    for (int32_t p : s.pages) {
        if (--pool->ref[p] == 0) pool->free_stack.push_back(p);
    }
    s.pages = std::move(slots);
    s.swapped = true;
    pool->n_swapped += 1;
    *n_pairs_out = n;
    return PA_OK;
}

pa_status pa_seq_swap_in(pa_pool* pool, int32_t seq, int32_t* pairs_out, int32_t max_pairs,
                         int32_t* n_pairs_out) {
    if (!pool || !n_pairs_out) return fail(PA_ERR_INVALID, "pa_seq_swap_in: null argument");
    if (!pool->in_use(seq) || !pool->seqs[seq].swapped)
        return fail(PA_ERR_STATE, "pa_seq_swap_in: sequence is not swapped out");
    auto& s = pool->seqs[seq];
    const int32_t n = (int32_t)s.pages.size();
    if (n > max_pairs || (n > 0 && !pairs_out))
        return fail(PA_ERR_INVALID, "pa_seq_swap_in: pairs_out too small");
    if (n > (int32_t)pool->free_stack.size())
        return fail(PA_ERR_NO_PAGES, "pa_seq_swap_in: page pool exhausted");
    std::vector<int32_t> pages(n);
    for (int32_t j = 0; j < n; ++j) {
        pages[j] = pool->pop();
        pool->ref[pages[j]] = 1;
        pairs_out[2 * j] = s.pages[j];
        pairs_out[2 * j + 1] = pages[j];
    }
    for (int32_t h : s.pages) pool->host_free.push_back(h);
    s.pages = std::move(pages);
    s.swapped = false;
    pool->n_swapped -= 1;
    *n_pairs_out = n;
    return PA_OK;
}

pa_status pa_pool_compact(pa_pool* pool, int32_t* pairs_out, int32_t max_pairs, int32_t* n_pairs_out) {
    if (!pool || !n_pairs_out) return fail(PA_ERR_INVALID, "pa_pool_compact: null argument");
    int32_t n_live = 0;
    for (int32_t r : pool->ref) n_live += r > 0;
    std::vector<int32_t> movers, holes;
    for (int32_t p = n_live; p < pool->num_pages; ++p)
        if (pool->ref[p] > 0) movers.push_back(p);
    for (int32_t p = 0; p < n_live; ++p)
        if (pool->ref[p] == 0) holes.push_back(p);
    const int32_t n = (int32_t)movers.size();
    if (n > max_pairs || (n > 0 && !pairs_out))
        return fail(PA_ERR_INVALID, "pa_pool_compact: pairs_out too small");
    std::vector<int32_t> dest(pool->num_pages);
    for (int32_t p = 0; p < pool->num_pages; ++p) dest[p] = p;
    for (int32_t i = 0; i < n; ++i) {
        dest[movers[i]] = holes[i];
        pairs_out[2 * i] = movers[i];
        pairs_out[2 * i + 1] = holes[i];
    }
    for (auto& s : pool->seqs)
        if (s.live && !s.swapped)
            for (int32_t& p : s.pages) p = dest[p];
    std::fill(pool->node_of_page.begin(), pool->node_of_page.end(), -1);
    for (size_t n = 1; n < pool->nodes.size(); ++n) {
        auto& x = pool->nodes[n];
        if (x.page < 0) continue;
        x.page = dest[x.page];
        pool->node_of_page[x.page] = (int32_t)n;
    }
    for (int32_t i = 0; i < n; ++i) {
        pool->ref[holes[i]] = pool->ref[movers[i]];
        pool->ref[movers[i]] = 0;
    }
    pool->free_stack.clear();
    for (int32_t p = pool->num_pages - 1; p >= n_live; --p) pool->free_stack.push_back(p);
    *n_pairs_out = n;
    return PA_OK;
}

pa_status pa_pool_host_stats(const pa_pool* pool, int32_t* n_host_free_out) {
    if (!pool || !n_host_free_out) return fail(PA_ERR_INVALID, "pa_pool_host_stats: null argument");
    *n_host_free_out = (int32_t)pool->host_free.size();
    return PA_OK;
}

pa_status pa_prefix_capacity(pa_pool* pool, int32_t max_pages, int32_t* n_freed_out) {
    if (!pool || max_pages < 0) return fail(PA_ERR_INVALID, "pa_prefix_capacity: bad argument");
    pool->capacity = max_pages;
    int32_t freed = pool->evict_over_capacity();
    if (n_freed_out) *n_freed_out = freed;
    return PA_OK;
}

pa_status pa_prefix_insert(pa_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                           int32_t* n_cached_out) {
    if (!pool || n_tokens < 0 || (n_tokens > 0 && !tokens))
        return fail(PA_ERR_INVALID, "pa_prefix_insert: bad argument");
    if (!pool->live(seq)) return fail(PA_ERR_STATE, "pa_prefix_insert: sequence is not live");
    const auto& s = pool->seqs[seq];
    if (n_tokens > s.len)
        return fail(PA_ERR_INVALID, "pa_prefix_insert: more tokens than the sequence holds");
    const int32_t P = pool->page_size;
    const int32_t full = n_tokens / P;
    std::vector<int32_t> path;
    int32_t node = 0;
    int32_t j = 0;
    for (; j < full; ++j) {
        int32_t nx = pool->find_child(node, tokens + (int64_t)j * P);
        if (nx < 0) break;
        path.push_back(nx);
        node = nx;
    }
    for (int32_t k = j; k < full; ++k)
        if (pool->node_of_page[s.pages[k]] >= 0)
            return fail(PA_ERR_INVALID, "pa_prefix_insert: page already cached under another prefix");
    const uint64_t c = pool->clock++;
    for (int32_t n : path) pool->restamp(n, c);
    for (; j < full; ++j) {
        node = pool->add_node(node, tokens + (int64_t)j * P, s.pages[j], c);
        path.push_back(node);
    }
    pool->evict_over_capacity();
    if (n_cached_out) *n_cached_out = (int32_t)path.size();
    return PA_OK;
}

pa_status pa_prefix_match(pa_pool* pool, const int32_t* tokens, int32_t n_tokens, int32_t* seq_out,
                          int32_t* n_matched_out) {
    if (!pool || !seq_out || !n_matched_out || n_tokens < 0 || (n_tokens > 0 && !tokens))
        return fail(PA_ERR_INVALID, "pa_prefix_match: bad argument");
    const int32_t P = pool->page_size;
    std::vector<int32_t> path;
    int32_t node = 0;
    for (int32_t j = 0; j < n_tokens / P; ++j) {
        int32_t nx = pool->find_child(node, tokens + (int64_t)j * P);
        if (nx < 0) break;
        path.push_back(nx);
        node = nx;
    }
    const uint64_t c = pool->clock++;
    for (int32_t n : path) pool->restamp(n, c);
    int32_t id = pool->new_id();
    auto& d = pool->seqs[id];
    d.live = true;
    d.swapped = false;
    d.pages.clear();
    for (int32_t n : path) {
        int32_t p = pool->nodes[n].page;
        d.pages.push_back(p);
        pool->ref[p] += 1;
    }
    d.len = (int64_t)path.size() * P;
    *seq_out = id;
    *n_matched_out = (int32_t)d.len;
    return PA_OK;
}

pa_status pa_prefix_evict(pa_pool* pool, int32_t n_pages, int32_t* n_freed_out) {
    if (!pool || !n_freed_out || n_pages < 0) return fail(PA_ERR_INVALID, "pa_prefix_evict: bad argument");
    const size_t target = pool->free_stack.size() + (size_t)n_pages;
    *n_freed_out = pool->evict([pool, target] { return pool->free_stack.size() < target; });
    return PA_OK;
}

pa_status pa_prefix_stats(const pa_pool* pool, int32_t* n_cached_out) {
    if (!pool || !n_cached_out) return fail(PA_ERR_INVALID, "pa_prefix_stats: null argument");
    *n_cached_out = pool->n_cached;
    return PA_OK;
}

}  // extern "C"
