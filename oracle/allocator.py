"""Oracle page pool: the allocation policy the host library must reproduce exactly.

The pages fix the structure (fixed-size blocks mapped through a per-sequence
block table, copy-on-write sharing -- page "CacheFlow：基于 llama.cpp 的多请求 LLM
推理优化引擎", section 2; a per-sequence page mapping plus true length -- page
"面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化", section 作品简介;
read-only shared prefixes with private suffixes and accounting over the union of
physical cells -- page "面向边缘智能体推理的 llama.cpp KV Cache 共享与复用优化",
section 主要功能与技术路线).  They leave the choice of *which* free page to use
open; this model fixes it so block tables are unique:

* the free list is a stack; initially ``free_order[0]`` is on top, so pages are
  handed out in ``free_order`` order;
* a page whose reference count drops to 0 is pushed on top (freed in logical
  page order);
* append fills the last page before taking a new one; if the last page is
  shared (refcount > 1) and partially filled, appending first gives the
  sequence a private copy of it (copy-on-write) and reports the (src, dst) pair;
* fork shares every page of the source (refcount + 1 each);
* cow of a logical page takes one new page, repoints the table entry, and drops
  the old page's refcount; it is an error on an unshared page;
* sequence ids are the smallest non-negative integer not in use;
* a failing call leaves the pool unchanged.

Preemption and compaction (page "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化
引擎", sections 内存管理策略 and 抢占与恢复机制: a preempted sequence's blocks go to a
reserved CPU area and come back without recomputation; fragmented blocks are
moved into contiguous physical locations).  The pages fix neither the slot
choice nor the move order; this model fixes them:

* the host reserve is ``n_host`` page slots kept as a second stack (slot 0 on
  top); swap-out gives each page of the sequence, in logical order, a host
  slot and drops the sequence's reference on the device page (pages whose
  count reaches 0 are pushed like ``seq_free`` does); swap-in takes a device
  page per host slot, in logical order, and pushes the host slots back in
  logical order.  A swapped-out sequence keeps its id; only ``seq_free`` and
  ``seq_swap_in`` accept it;
* compaction with ``n_live`` pages in use moves every live page whose id is
  >= ``n_live`` (ascending) onto the free ids below ``n_live`` (ascending),
  carries refcounts and table entries along (prefix-index pages included), and
  rebuilds the free stack as ``n_live .. N-1`` with ``n_live`` on top.

Prefix cache (page "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎", section
核心架构与技术贡献 item 2 and section 前缀缓存优化: a trie lookup reuses the blocks of
shared prefixes; page "面向边缘智能体推理的 llama.cpp KV Cache 共享与复用优化",
section 主要功能与技术路线: longest-prefix match over a token prefix tree, with LRU
reclaim of its leaves).  Page-aligned reading: the tree's edges are whole pages
of token ids, since a page is the unit that two sequences can share without a
copy; each node holds one physical page and one reference on it.

* ``prefix_insert(seq, tokens)`` walks the sequence's full pages (tokens
  ``jP .. jP+P-1`` for ``(j+1)P <= len(tokens)``, which must not exceed the
  sequence's length); a missing node takes the sequence's page ``j`` (ref + 1),
  an existing node keeps its page; every node on the path gets the current
  clock value, then the clock advances;
* ``prefix_match(tokens)`` follows full pages as far as they match, stamps the
  matched path, advances the clock and returns a new sequence sharing those
  pages (ref + 1 each) with length ``matched_pages * P``;
* when more than ``capacity`` pages are cached (after an insert), and on
  ``prefix_evict(n)``, the leaf with the oldest stamp is removed (its index
  reference dropped, the page pushed if its count reaches 0), repeatedly;
  stamps of leaves are unique because one call stamps one path.

Pinned by invariants (page conservation, sharing only under refcount > 1,
free-all restores every page, page counts with and without sharing) in
tests/test_oracle.py.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


class PoolError(Exception):
    status = -1


class InvalidError(PoolError):
    status = -1


class NoPagesError(PoolError):
    status = -3


class StateError(PoolError):
    status = -4


class AllocatorModel:
    def __init__(self, num_pages: int, page_size: int, free_order: Optional[Sequence[int]] = None):
        if num_pages < 1 or page_size < 1:
            raise InvalidError("bad pool size")
        order = list(range(num_pages)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_pages)):
            raise InvalidError("free_order must be a permutation of 0..N-1")
        self.num_pages = num_pages
        self.page_size = page_size
        self.free: List[int] = order[::-1]          # top of stack = end of list
        self.ref = [0] * num_pages
        self.pages: Dict[int, List[int]] = {}
        self.length: Dict[int, int] = {}
        self.host: Dict[int, List[int]] = {}         # swapped-out sequences' host slots
        self.host_free: List[int] = []
        self.n_host = 0
        # prefix trie: node id -> [parent, key tuple, page, stamp]; children by (parent, key)
        self.trie: Dict[int, list] = {}
        self.child: Dict[Tuple[int, tuple], int] = {}
        self.next_node = 1                           # node 0 is the root
        self.clock = 0
        self.capacity = num_pages

    # -- helpers
    def _pop(self) -> int:
        return self.free.pop()

    def _alive(self, seq: int):
        if seq not in self.pages:
            raise StateError(f"sequence {seq} is not live (or is swapped out)")

    # -- API mirror
    def seq_new(self) -> int:
        sid = 0
        while sid in self.pages or sid in self.host:
            sid += 1
        self.pages[sid] = []
        self.length[sid] = 0
        return sid

    def seq_append(self, seq: int, n_new: int) -> Tuple[np.ndarray, Optional[Tuple[int, int]]]:
        self._alive(seq)
        if n_new < 0:
            raise InvalidError("n_new < 0")
        P = self.page_size
        L = self.length[seq]
        pages = self.pages[seq]
        if n_new == 0:
            return np.zeros(0, dtype=np.int32), None
        cow = bool(L % P) and self.ref[pages[-1]] > 1
        need = (L + n_new + P - 1) // P - (L + P - 1) // P + (1 if cow else 0)
        if need > len(self.free):
            raise NoPagesError("pool exhausted")
        pair = None
        if cow:
            src = pages[-1]
            dst = self._pop()
            self.ref[src] -= 1
            self.ref[dst] = 1
            pages[-1] = dst
            pair = (src, dst)
        slots = np.empty(n_new, dtype=np.int32)
        for j in range(n_new):
            t = L + j
            if t % P == 0:
                p = self._pop()
                self.ref[p] = 1
                pages.append(p)
            slots[j] = pages[t // P] * P + t % P
        self.length[seq] = L + n_new
        return slots, pair

    def seq_fork(self, src: int) -> int:
        self._alive(src)
        dst = self.seq_new()
        self.pages[dst] = list(self.pages[src])
        self.length[dst] = self.length[src]
        for p in self.pages[dst]:
            self.ref[p] += 1
        return dst

    def seq_cow(self, seq: int, logical_page: int) -> Tuple[int, int]:
        self._alive(seq)
        pages = self.pages[seq]
        if logical_page < 0 or logical_page >= len(pages):
            raise InvalidError("logical page out of range")
        src = pages[logical_page]
        if self.ref[src] < 2:
            raise StateError("page is not shared")
        if not self.free:
            raise NoPagesError("pool exhausted")
        dst = self._pop()
        self.ref[src] -= 1
        self.ref[dst] = 1
        pages[logical_page] = dst
        return src, dst

    def seq_free(self, seq: int) -> None:
        if seq in self.host:
            for h in self.host[seq]:
                self.host_free.append(h)
            del self.host[seq]
            del self.length[seq]
            return
        self._alive(seq)
        for p in self.pages[seq]:
            self.ref[p] -= 1
            if self.ref[p] == 0:
                self.free.append(p)
        del self.pages[seq]
        del self.length[seq]

    def block_tables(self, seqs: Sequence[int], max_pages: int):
        for s in seqs:
            self._alive(s)
            if len(self.pages[s]) > max_pages:
                raise InvalidError("max_pages too small")
        bt = np.full((len(seqs), max_pages), -1, dtype=np.int32)
        kv = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            bt[i, :len(self.pages[s])] = self.pages[s]
            kv[i] = self.length[s]
        return bt, kv

    def stats(self):
        return len(self.free), np.asarray(self.ref, dtype=np.int32)

    # -- preemption: swap to / from the host reserve
    def host_reserve(self, n_host: int) -> None:
        if n_host < 0:
            raise InvalidError("n_host < 0")
        if self.host:
            raise StateError("sequences are swapped out")
        self.n_host = n_host
        self.host_free = list(range(n_host))[::-1]   # slot 0 on top

    def seq_swap_out(self, seq: int) -> List[Tuple[int, int]]:
        """Returns the (device page, host slot) copies to make, in logical order."""
        self._alive(seq)
        pages = self.pages[seq]
        if len(pages) > len(self.host_free):
            raise NoPagesError("host reserve exhausted")
        pairs = []
        slots = []
        for p in pages:
            h = self.host_free.pop()
            pairs.append((p, h))
            slots.append(h)
        for p in pages:
            self.ref[p] -= 1
            if self.ref[p] == 0:
                self.free.append(p)
        del self.pages[seq]
        self.host[seq] = slots
        return pairs

    def seq_swap_in(self, seq: int) -> List[Tuple[int, int]]:
        """Returns the (host slot, device page) copies to make, in logical order."""
        if seq not in self.host:
            raise StateError("sequence is not swapped out")
        slots = self.host[seq]
        if len(slots) > len(self.free):
            raise NoPagesError("pool exhausted")
        pairs = []
        pages = []
        for h in slots:
            p = self._pop()
            self.ref[p] = 1
            pairs.append((h, p))
            pages.append(p)
        for h in slots:
            self.host_free.append(h)
        del self.host[seq]
        self.pages[seq] = pages
        return pairs

    # -- compaction
    def compact(self) -> List[Tuple[int, int]]:
        """Moves live pages into ids 0..n_live-1; returns the (src, dst) copies."""
        n_live = sum(1 for r in self.ref if r > 0)
        movers = [p for p in range(n_live, self.num_pages) if self.ref[p] > 0]
        holes = [p for p in range(n_live) if self.ref[p] == 0]
        assert len(movers) == len(holes)
        dest = dict(zip(movers, holes))
        for s in self.pages:
            self.pages[s] = [dest.get(p, p) for p in self.pages[s]]
        for node in self.trie.values():
            node[2] = dest.get(node[2], node[2])
        for src, dst in dest.items():
            self.ref[dst] = self.ref[src]
            self.ref[src] = 0
        self.free = list(range(n_live, self.num_pages))[::-1]
        return list(zip(movers, holes))

    def stats_host(self):
        return len(self.host_free)

    # -- prefix cache
    def prefix_capacity(self, max_pages: int) -> int:
        """Sets the cached-page budget; returns the pages freed to meet it."""
        if max_pages < 0:
            raise InvalidError("capacity < 0")
        self.capacity = max_pages
        return self._evict(lambda: len(self.trie) > self.capacity)

    def _evict(self, more) -> int:
        """Removes least recently stamped evictable leaves while more() holds.
        A leaf is evictable when the index's reference is its page's only one,
        so every removal frees exactly one page."""
        freed = 0
        while more():
            parents = {v[0] for v in self.trie.values()}
            cand = [n for n, v in self.trie.items() if n not in parents and self.ref[v[2]] == 1]
            if not cand:
                break
            n = min(cand, key=lambda x: self.trie[x][3])
            parent, key, page, _ = self.trie.pop(n)
            del self.child[(parent, key)]
            self.ref[page] = 0
            self.free.append(page)
            freed += 1
        return freed

    def prefix_insert(self, seq: int, tokens: Sequence[int]) -> int:
        """Returns the number of pages cached along the sequence's path."""
        self._alive(seq)
        P = self.page_size
        tokens = [int(t) for t in tokens]
        if len(tokens) > self.length[seq]:
            raise InvalidError("more tokens than the sequence holds")
        cached = {v[2] for v in self.trie.values()}
        node, path, new = 0, [], []
        for j in range(len(tokens) // P):
            key = tuple(tokens[j * P:(j + 1) * P])
            nxt = self.child.get((node, key)) if node >= 0 else None
            if nxt is None:
                page = self.pages[seq][j]
                if page in cached:
                    raise InvalidError("page already cached under another prefix")
                new.append((j, key))
                node = -1
            else:
                path.append(nxt)
                node = nxt
        node = path[-1] if path else 0
        for j, key in new:
            nxt = self.next_node
            self.next_node += 1
            page = self.pages[seq][j]
            self.ref[page] += 1
            self.trie[nxt] = [node, key, page, 0]
            self.child[(node, key)] = nxt
            path.append(nxt)
            node = nxt
        for n in path:
            self.trie[n][3] = self.clock
        self.clock += 1
        self._evict(lambda: len(self.trie) > self.capacity)
        return len(path)

    def prefix_match(self, tokens: Sequence[int]) -> Tuple[int, int]:
        """Returns (new sequence sharing the longest cached page-aligned prefix,
        matched tokens)."""
        P = self.page_size
        tokens = [int(t) for t in tokens]
        node, path = 0, []
        for j in range(len(tokens) // P):
            nxt = self.child.get((node, tuple(tokens[j * P:(j + 1) * P])))
            if nxt is None:
                break
            path.append(nxt)
            node = nxt
        for n in path:
            self.trie[n][3] = self.clock
        self.clock += 1
        seq = self.seq_new()
        pages = [self.trie[n][2] for n in path]
        for p in pages:
            self.ref[p] += 1
        self.pages[seq] = pages
        self.length[seq] = len(pages) * P
        return seq, len(pages) * P

    def prefix_evict(self, n_pages: int) -> int:
        """Frees up to n_pages cached pages in LRU order; returns how many."""
        if n_pages < 0:
            raise InvalidError("n_pages < 0")
        target = len(self.free) + n_pages
        return self._evict(lambda: len(self.free) < target)

    def prefix_pages(self) -> int:
        return len(self.trie)
