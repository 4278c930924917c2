"""Oracle attention: dense per-sequence causal softmax attention, float64.

UA-PagedAttention (page "面向多并发长上下文的 llama.cpp 分页式 KV Cache 与计算加速优化",
section 作品简介) reaches the same result as masked attention over a unified
cache; it only avoids touching positions the mask excludes.  The oracle is
therefore the plain definition, computed over the logically concatenated valid
pages of each query's own sequence:

    n_i        = min(kv_len_i, pos_i + 1)
    z_t        = scale * <q_{i,h}, K_t[h // G]>          for t < n_i
    out_{i,h}  = sum_t exp(z_t - max z) V_t[h // G]  /  sum_t exp(z_t - max z)

with G = Hq / Hkv (query head h reads KV head h // G).  Pool storage: K is
``[N][Hkv][P][D]`` and V is ``[N][Hkv][P // B][D][B]`` with B = min(P, 32): the
value column of slot s of page p, KV head h, is ``V[p, h, s // B, :, s % B]``.
Logical cell t of a sequence is page ``table[t // P]``, slot ``t % P``.
"""
from __future__ import annotations

import math

import numpy as np


def v_block(page_size: int) -> int:
    """Slots per block of a V page: the V storage convention above."""
    return min(int(page_size), 32)


def check_v_pool(k_pool: np.ndarray, v_pool: np.ndarray) -> int:
    """Check that ``v_pool`` has the V storage shape that goes with ``k_pool``;
    return the block size B."""
    num_pages, n_kv, page_size, head_dim = k_pool.shape
    B = v_block(page_size)
    want = (num_pages, n_kv, page_size // B, head_dim, B)
    if tuple(v_pool.shape) != want:
        raise ValueError(f"V pool shape {tuple(v_pool.shape)} is not {want}")
    return B


def expand_per_token(block_tables: np.ndarray, token_row: np.ndarray) -> np.ndarray:
    """UA expansion: every ubatch token carries its own sequence's block-table row,
    in token order (page above, section 作品简介).  Padding tokens (row -1) get an
    all -1 row.  Returns int64 ``[T][max_pages]``."""
    bt = np.asarray(block_tables)
    rows = np.asarray(token_row)
    out = np.full((rows.shape[0], bt.shape[1]), -1, dtype=np.int64)
    for i, r in enumerate(rows):
        if r >= 0:
            out[i] = bt[r]
    return out


def gather_logical(k_pool: np.ndarray, v_pool: np.ndarray, pages: np.ndarray, n: int):
    """Logical K and V of cells 0..n-1 of one sequence, as float64 ``[n][Hkv][D]``.

    Only the ceil(n / P) pages that hold those cells are read; each page id must be
    a real page of the pool."""
    num_pages, n_kv, page_size, head_dim = k_pool.shape
    check_v_pool(k_pool, v_pool)
    n_pages = (n + page_size - 1) // page_size
    ids = np.asarray(pages[:n_pages], dtype=np.int64)
    if ids.shape[0] != n_pages or np.any(ids < 0) or np.any(ids >= num_pages):
        raise ValueError("block table does not cover the requested cells")
    k = k_pool[ids]                                  # [np][Hkv][P][D]
    v = v_pool[ids]                                  # [np][Hkv][P/B][D][B]
    k = k.transpose(0, 2, 1, 3).reshape(n_pages * page_size, n_kv, head_dim)[:n]
    # cell order: page, then slot block, then slot in the block
    v = v.transpose(0, 2, 4, 1, 3).reshape(n_pages * page_size, n_kv, head_dim)[:n]
    return k.astype(np.float64), v.astype(np.float64)


def paged_attention(q, k_pool, v_pool, block_tables, token_row, token_kv_len, token_pos,
                    scale) -> np.ndarray:
    """Attention for a ubatch whose tokens each carry (table row, true KV length,
    position).  ``q`` is ``[T][Hq][D]``; returns float64 ``[T][Hq][D]``.  A token
    with row -1 is padding and gets a zero row.

    Pinned by: brute-force triple loop over the physical pool, torch CPU float64
    scaled_dot_product_attention on single-page inputs, closed forms, page
    permutation and NaN-poison invariance (tests/test_oracle.py)."""
    q = np.asarray(q)
    T, n_q, head_dim = q.shape
    n_kv = k_pool.shape[1]
    if n_q % n_kv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = n_q // n_kv
    scale64 = float(np.float32(scale))
    rows = np.asarray(token_row, dtype=np.int64)
    kv_len = np.asarray(token_kv_len, dtype=np.int64)
    pos = np.asarray(token_pos, dtype=np.int64)
    bt_tok = expand_per_token(block_tables, rows)
    out = np.zeros((T, n_q, head_dim), dtype=np.float64)
    n_tok = np.minimum(kv_len, pos + 1)
    q64 = q.astype(np.float64)
    # Tokens of one sequence carry identical expanded rows; gather that sequence's
    # cells once (up to the longest any of its tokens needs) and slice per token.
    for r in np.unique(rows[rows >= 0]):
        idx = np.nonzero(rows == r)[0]
        if np.any(n_tok[idx] < 1):
            raise ValueError("a query token must see at least one key")
        n_max = int(n_tok[idx].max())
        K, V = gather_logical(k_pool, v_pool, bt_tok[idx[0]], n_max)
        for i in idx:
            n = int(n_tok[i])
            for g in range(n_kv):
                Kg = K[:n, g, :]                        # [n][D]
                Vg = V[:n, g, :]
                Qg = q64[i, g * G:(g + 1) * G, :]       # [G][D]
                z = scale64 * (Qg @ Kg.T)               # [G][n]
                z -= z.max(axis=1, keepdims=True)
                w = np.exp(z)
                out[i, g * G:(g + 1) * G, :] = (w @ Vg) / w.sum(axis=1, keepdims=True)
    return out


def paged_decode(q, k_pool, v_pool, block_tables, kv_lens, scale) -> np.ndarray:
    """Decode: one query per sequence at position kv_len-1, i.e. the UA case with
    token i = sequence i.  Returns float64 ``[S][Hq][D]``."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    S = kv_lens.shape[0]
    return paged_attention(q, k_pool, v_pool, block_tables, np.arange(S), kv_lens, kv_lens - 1,
                           scale)


def partitioned_decode(q, k_pool, v_pool, block_tables, kv_lens, scale, partition_tokens):
    """Split-KV decode (page "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎",
    section 3, the partition-plus-reduce kernel for long contexts).

    Each sequence's cells are cut into partitions of ``partition_tokens``; for each
    partition p and query head: m_p = max z, l_p = sum exp(z - m_p),
    acc_p = sum exp(z - m_p) V.  Returns (out, m, l, acc) with m, l
    ``[S][Hq][n_part]`` (unused partitions: m = -inf, l = 0) and acc
    ``[S][Hq][n_part][D]``.  ``out`` comes from :func:`lse_combine`.

    Pinned by equality with :func:`paged_decode` (exact identity up to rounding)."""
    q = np.asarray(q)
    S, n_q, head_dim = q.shape
    n_kv = k_pool.shape[1]
    G = n_q // n_kv
    scale64 = float(np.float32(scale))
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    n_part = int(max(1, max((int(L) + partition_tokens - 1) // partition_tokens for L in kv_lens)))
    m = np.full((S, n_q, n_part), -np.inf)
    l = np.zeros((S, n_q, n_part))
    acc = np.zeros((S, n_q, n_part, head_dim))
    for s in range(S):
        L = int(kv_lens[s])
        K, V = gather_logical(k_pool, v_pool, np.asarray(block_tables)[s], L)
        for p in range((L + partition_tokens - 1) // partition_tokens):
            a, b = p * partition_tokens, min(L, (p + 1) * partition_tokens)
            for h in range(n_q):
                g = h // G
                z = scale64 * (K[a:b, g, :] @ q[s, h].astype(np.float64))
                mp = z.max()
                w = np.exp(z - mp)
                m[s, h, p] = mp
                l[s, h, p] = w.sum()
                acc[s, h, p] = w @ V[a:b, g, :]
    return lse_combine(m, l, acc), m, l, acc


def lse_combine(m, l, acc):
    """Log-sum-exp combine of partitions: M = max_p m_p, w_p = exp(m_p - M),
    out = sum_p w_p acc_p / sum_p w_p l_p.  Partitions with m = -inf weigh 0."""
    M = m.max(axis=-1, keepdims=True)
    w = np.where(np.isneginf(m), 0.0, np.exp(m - M))
    num = np.einsum("shp,shpd->shd", w, acc)
    den = np.einsum("shp,shp->sh", w, l)
    return num / den[..., None]


def unified_attention(q, k_pool, v_pool, span, cell_seq, cell_pos, token_seq, token_pos,
                      scale) -> np.ndarray:
    """Masked attention over one unified cache span (page "面向多并发长上下文的
    llama.cpp 分页式 KV Cache 与计算加速优化", section 作品简介: the original cache
    the method replaces, where every query of a ubatch faces one physical span
    of cells from all sequences, free cells and padding, and the mask excludes
    what does not belong to it).

    The span is cells 0..span-1 of the pool read as one flat array: cell c is
    page c // P, slot c % P.  Cell c holds position ``cell_pos[c]`` of sequence
    ``cell_seq[c]`` (-1: free or padding).  Token i (sequence ``token_seq[i]``,
    -1 = padding, position ``token_pos[i]``) sees exactly the cells with
    ``cell_seq == token_seq[i]`` and ``cell_pos <= token_pos[i]``; the result is
    softmax attention over those cells, float64 ``[T][Hq][D]``.  Padding tokens
    and tokens that see no cell get a zero row.

    Pinned by: equality with :func:`paged_attention` on the span view of paged
    cases (table gather against masked scan), a pure-Python brute force, and
    invariance to NaN in free cells and to page order (tests/test_oracle.py)."""
    q = np.asarray(q)
    T, n_q, head_dim = q.shape
    num_pages, n_kv, page_size, _ = k_pool.shape
    B = check_v_pool(k_pool, v_pool)
    G = n_q // n_kv
    span = int(span)
    if span > num_pages * page_size:
        raise ValueError("span exceeds the pool")
    scale64 = float(np.float32(scale))
    cseq = np.asarray(cell_seq, dtype=np.int64)[:span]
    cpos = np.asarray(cell_pos, dtype=np.int64)[:span]
    cells = np.arange(span)
    q64 = q.astype(np.float64)
    out = np.zeros((T, n_q, head_dim), dtype=np.float64)
    for i in range(T):
        s, p = int(token_seq[i]), int(token_pos[i])
        if s < 0:
            continue
        vis = cells[(cseq == s) & (cpos <= p)]
        if vis.size == 0:
            continue
        K = k_pool[vis // page_size, :, vis % page_size, :].astype(np.float64)   # [n][Hkv][D]
        slot = vis % page_size
        V = v_pool[vis // page_size, :, slot // B, :, slot % B].astype(np.float64)   # [n][Hkv][D]
        for g in range(n_kv):
            Qg = q64[i, g * G:(g + 1) * G, :]
            z = scale64 * (Qg @ K[:, g, :].T)
            z -= z.max(axis=1, keepdims=True)
            w = np.exp(z)
            out[i, g * G:(g + 1) * G, :] = (w @ V[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out
