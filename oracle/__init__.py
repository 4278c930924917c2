"""CPU oracle for paged attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It is plain numpy in float64, written from
the method as the pages state it and sharing no code with the HIP path.

Pages cited (titles as published):

* "面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化" -- the
  UA-PagedAttention page.  Section 作品简介: with a unified cache, attention
  still loads and computes the masked positions of other sequences, free cells
  and padding; the paged design keeps a page mapping and a true KV length per
  sequence, expands both per query token in ubatch order, and lets each query
  read only its own sequence's valid pages.
* "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎" -- section 2 (fixed-size
  blocks, block-table mapping, copy-on-write sharing), section 3 (V1 one-pass
  and V2 partition-plus-reduce attention kernels, reshape-and-cache, block copy).
* "面向边缘智能体推理的 llama.cpp KV Cache 共享与复用优化" -- section
  主要功能与技术路线 (a shared prefix is read-only; private suffixes are
  allocated per request; accounting is over the union of physical cells).

Pinning status of each function is given in its docstring; every function here
is pinned by tests that do not re-type its formula (brute force, library
routines, closed forms, invariants).
"""
from .attention import (expand_per_token, gather_logical, paged_attention, paged_decode,
                        partitioned_decode, lse_combine, unified_attention)
from .cache_ops import reshape_and_cache, copy_blocks, swap_blocks
from .allocator import AllocatorModel, PoolError, NoPagesError, StateError, InvalidError

__all__ = [
    "expand_per_token", "gather_logical", "paged_attention", "paged_decode",
    "partitioned_decode", "lse_combine", "unified_attention", "reshape_and_cache", "copy_blocks", "swap_blocks",
    "AllocatorModel", "PoolError", "NoPagesError", "StateError", "InvalidError",
]
