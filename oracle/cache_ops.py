"""Oracle cache operations: reshape-and-cache and block copy.

Both are listed as fused kernels on page "CacheFlow：基于 llama.cpp 的多请求 LLM
推理优化引擎", section 3 (reshape-and-cache writes new tokens' K/V into their
blocks; block copy serves copy-on-write sharing, section 2).  Results are
defined bit for bit: values are moved, never recomputed, except that a float32
source is rounded to float16 by numpy (IEEE round to nearest even).
"""
from __future__ import annotations

import numpy as np


def reshape_and_cache(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Return copies of the pools with token i's K/V written to cell
    ``slot_mapping[i]`` (page = slot // P, slot-in-page = slot % P).  Negative slots
    are skipped.  ``k_new``/``v_new`` are ``[T][Hkv][D]`` float16 or float32.

    Pinned by: byte-level checks that only the addressed cells change and hold
    the source bits (tests/test_oracle.py), and numpy's own IEEE rounding."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    page_size = k_out.shape[2]
    B = min(page_size, 32)   # V pages hold their slots in blocks of B, slot innermost
    if tuple(v_out.shape) != (k_out.shape[0], k_out.shape[1], page_size // B, k_out.shape[3], B):
        raise ValueError("V pool shape does not match the K pool")
    kn = np.asarray(k_new)
    vn = np.asarray(v_new)
    if kn.dtype != np.float16:
        kn = kn.astype(np.float16)
    if vn.dtype != np.float16:
        vn = vn.astype(np.float16)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = slots[slots >= 0]
    if np.unique(live).shape[0] != live.shape[0]:
        raise ValueError("slot_mapping must not repeat a slot")
    for i, s in enumerate(slots):
        if s < 0:
            continue
        page, off = int(s) // page_size, int(s) % page_size
        k_out[page, :, off, :] = kn[i]
        v_out[page, :, off // B, :, off % B] = vn[i]
    return k_out, v_out


def copy_blocks(k_pools, v_pools, pairs):
    """Copy whole physical pages src -> dst in every layer's K and V pool.

    ``k_pools``/``v_pools`` are lists (one pool per layer); returns new lists.
    A destination may appear once and may not also be a source, so the result
    does not depend on the order of the pairs."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    dst = pairs[:, 1]
    if np.unique(dst).shape[0] != dst.shape[0] or np.intersect1d(dst, pairs[:, 0]).size:
        raise ValueError("copy_blocks: a destination repeats or is also a source")
    ks = [np.array(k, copy=True) for k in k_pools]
    vs = [np.array(v, copy=True) for v in v_pools]
    for layer in range(len(ks)):
        for s, d in pairs:
            ks[layer][d] = k_pools[layer][s]
            vs[layer][d] = v_pools[layer][s]
    return ks, vs


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """Copy whole pages from one pool pair to another of the same page layout
    (page "CacheFlow：基于 llama.cpp 的多请求 LLM 推理优化引擎", section 3, the block
    swap between GPU and CPU memory): ``dst[d] = src[s]`` for every (s, d) pair
    and every layer.  ``src_*``/``dst_*`` are lists (one pool per layer);
    returns new destination lists.  A destination may appear once, so the
    result does not depend on the order of the pairs."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    if np.unique(pairs[:, 1]).shape[0] != pairs.shape[0]:
        raise ValueError("swap_blocks: a destination repeats")
    ks = [np.array(k, copy=True) for k in dst_k]
    vs = [np.array(v, copy=True) for v in dst_v]
    for layer in range(len(ks)):
        for s, d in pairs:
            ks[layer][d] = src_k[layer][s]
            vs[layer][d] = src_v[layer][s]
    return ks, vs
