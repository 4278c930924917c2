"""Seeded generators for the five paged-attention workloads and their work counts.

Storage format of a cache pool (one layer), shared by every consumer:

* K pool: float16 ``[num_pages][n_kv_heads][page_size][head_dim]``
* V pool: float16 ``[num_pages][n_kv_heads][page_size // B][head_dim][B]`` with
  ``B = min(page_size, 32)``: a page's slots in blocks of B, each block slot
  innermost (for page_size <= 32 this is ``[num_pages][n_kv_heads][head_dim][page_size]``).
  V values are drawn as columns ``[num_pages][n_kv_heads][head_dim][page_size]``
  and then laid into this storage (``v_blocks_from_columns``), so what a seed
  gives does not depend on the storage layout.

A *cell* is one (page, slot) position.  Cells that hold no token of a live
sequence (free pages, padding after a sequence's last token, cells whose token
is still to be written) are filled with the float16 quiet NaN ``0x7E00`` so that
any read of them poisons an attention result.

Random draws use ``np.random.default_rng(185000 + c)`` for workload ``c`` and,
unless a generator says otherwise, happen in this order: physical page
permutation, lengths, Q, K, V.  Values are drawn in float32 and rounded to
float16 by numpy (round to nearest even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

NAN_F16_BITS = np.uint16(0x7E00)

__all__ = [
    "NAN_F16_BITS", "DecodeCase", "PrefillCase", "ChunkedPrefill", "SharingCase",
    "rng_for", "poison_pools", "v_block", "v_blocks_from_columns", "make_decode_case", "make_prefill_case",
    "tiny_decode", "qwen3_decode", "ua_prefill", "varlen_decode", "sharing_case",
    "chunked_prefill", "decode_valid_bytes", "attention_flops", "prefill_pairs",
    "fp32_scale",
]


def rng_for(config_index: int) -> np.random.Generator:
    return np.random.default_rng(185000 + config_index)


def fp32_scale(head_dim: int) -> np.float32:
    """Softmax scale 1/sqrt(head_dim), rounded once to float32."""
    return np.float32(1.0 / math.sqrt(head_dim))


def _normal(rng, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _normal_f16(rng, shape, std=1.0) -> np.ndarray:
    return _normal(rng, shape, std).astype(np.float16)


def poison_pools(k_pool: np.ndarray, v_pool: np.ndarray, valid_cells: np.ndarray) -> None:
    """Overwrite every cell that is not marked valid with float16 NaN, in place.

    ``valid_cells`` is bool ``[num_pages][page_size]``.
    """
    bad = ~valid_cells
    kb = k_pool.view(np.uint16)
    vb = v_pool.view(np.uint16)
    kb[np.broadcast_to(bad[:, None, :, None], kb.shape)] = NAN_F16_BITS
    n, _, nblk, _, blk = vb.shape
    vbad = bad.reshape(n, nblk, blk)   # slot s -> (block s // B, s % B)
    vb[np.broadcast_to(vbad[:, None, :, None, :], vb.shape)] = NAN_F16_BITS


def v_block(page_size: int) -> int:
    """Slots per block of a V page: V storage is [N][Hkv][P // B][D][B], B = min(P, 32)."""
    return min(int(page_size), 32)


def _pool_shapes(n_pages, n_kv_heads, page_size, head_dim):
    B = v_block(page_size)
    return ((n_pages, n_kv_heads, page_size, head_dim),
            (n_pages, n_kv_heads, page_size // B, head_dim, B))


def v_blocks_from_columns(v: np.ndarray) -> np.ndarray:
    """V pages given as value columns ``[N][Hkv][D][P]`` in V storage order
    ``[N][Hkv][P // B][D][B]``."""
    n, h, d, p = v.shape
    B = v_block(p)
    return np.ascontiguousarray(v.reshape(n, h, d, p // B, B).transpose(0, 1, 3, 2, 4))


def _draw_pools(rng, n_pages, n_kv_heads, page_size, head_dim, std):
    ks, _ = _pool_shapes(n_pages, n_kv_heads, page_size, head_dim)
    k = _normal_f16(rng, ks, std)
    # drawn as value columns [N][Hkv][D][P], then stored in V page order
    v = v_blocks_from_columns(_normal_f16(rng, (n_pages, n_kv_heads, head_dim, page_size), std))
    return k, v


def _assign_pages(perm: np.ndarray, lens, page_size: int, max_pages: Optional[int] = None):
    """Give sequence s the next ceil(len_s/page_size) ids of ``perm``; build the
    -1 padded block table and the valid-cell mask."""
    n_pages_each = [(int(L) + page_size - 1) // page_size for L in lens]
    mp = max(n_pages_each) if max_pages is None else max_pages
    bt = np.full((len(lens), max(mp, 1)), -1, dtype=np.int32)
    valid = np.zeros((len(perm), page_size), dtype=bool)
    cur = 0
    for s, L in enumerate(lens):
        k = n_pages_each[s]
        pages = perm[cur:cur + k]
        if len(pages) < k:
            raise ValueError("pool too small for the requested lengths")
        cur += k
        bt[s, :k] = pages
        for j, p in enumerate(pages):
            n_here = min(page_size, int(L) - j * page_size)
            valid[p, :n_here] = True
    return bt, valid


@dataclass
class DecodeCase:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    q: np.ndarray             # float32 [S][Hq][D]
    k_pool: np.ndarray        # float16 [N][Hkv][P][D]
    v_pool: np.ndarray        # float16 [N][Hkv][P // B][D][B], B = min(P, 32)
    block_tables: np.ndarray  # int32 [S][max_pages], -1 padded
    kv_lens: np.ndarray       # int32 [S]
    scale: np.float32
    valid_cells: np.ndarray = field(repr=False, default=None)

    @property
    def n_seqs(self):
        return self.q.shape[0]


def make_decode_case(rng, name, n_q_heads, n_kv_heads, head_dim, page_size, kv_lens,
                     num_pages, std=1.0, perm=None) -> DecodeCase:
    if perm is None:
        perm = rng.permutation(num_pages)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    bt, valid = _assign_pages(perm, kv_lens, page_size)
    q = _normal(rng, (len(kv_lens), n_q_heads, head_dim), std)
    k, v = _draw_pools(rng, num_pages, n_kv_heads, page_size, head_dim, std)
    poison_pools(k, v, valid)
    return DecodeCase(name, n_q_heads, n_kv_heads, head_dim, page_size, num_pages, q, k, v,
                      bt, kv_lens, fp32_scale(head_dim), valid)


def tiny_decode() -> DecodeCase:
    """1 layer, Hq 4, Hkv 2, D 64, P 16, pool of 64 permuted pages, lengths 37 and 200."""
    rng = rng_for(0)
    perm = rng.permutation(64)
    return make_decode_case(rng, "tiny_decode", 4, 2, 64, 16, [37, 200], 64, 1.0, perm)


def qwen3_decode(n_seqs=8, kv_len=16384, num_pages=2048) -> DecodeCase:
    """Hq 32, Hkv 8, D 128, P 128; 8 x 16384 tokens scattered in a 2048-page pool;
    values N(0,1)*0.5."""
    rng = rng_for(1)
    perm = rng.permutation(num_pages)
    return make_decode_case(rng, f"decode_{n_seqs}x{kv_len}_gqa32-8_d128_p128", 32, 8, 128, 128,
                            [kv_len] * n_seqs, num_pages, 0.5, perm)


def varlen_decode(page_size: int, n_seqs=64) -> DecodeCase:
    """64 sequences, lengths log-uniform in [256, 32768]; pool 1.25x the pages used.
    The lengths are drawn first here because the pool size depends on them."""
    rng = rng_for(3)
    u = rng.random(n_seqs)
    lens = np.clip(np.rint(256.0 * np.power(128.0, u)), 256, 32768).astype(np.int32)
    used = int(sum((int(L) + page_size - 1) // page_size for L in lens))
    n_pages = int(math.ceil(1.25 * used))
    perm = rng.permutation(n_pages)
    return make_decode_case(rng, f"varlen_decode_{n_seqs}_p{page_size}", 32, 8, 128, page_size,
                            lens, n_pages, 1.0, perm)


@dataclass
class PrefillCase:
    """One ubatch of query tokens from several sequences (UA-PagedAttention).

    ``k_pool``/``v_pool`` hold the pool *before* the ubatch's own K/V are
    written; those arrive in ``k_new``/``v_new`` with ``slot_mapping``.
    """
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    q: np.ndarray              # float32 [T][Hq][D]
    k_pool: np.ndarray         # float16 pool before the new tokens are cached
    v_pool: np.ndarray
    k_new: np.ndarray          # float16 [T][Hkv][D]
    v_new: np.ndarray
    slot_mapping: np.ndarray   # int32 [T] = page*P + offset
    block_tables: np.ndarray   # int32 [n_rows][max_pages]
    token_row: np.ndarray      # int32 [T]
    token_kv_len: np.ndarray   # int32 [T]
    token_pos: np.ndarray      # int32 [T]
    scale: np.float32
    seq_kv_lens: np.ndarray = None


def make_prefill_case(rng, name, n_q_heads, n_kv_heads, head_dim, page_size, num_pages,
                      prefixes, n_new, order="round_robin", std=1.0, perm=None) -> PrefillCase:
    """Sequences with ``prefixes[s]`` cached tokens each get ``n_new[s]`` new tokens.

    Draw order: permutation (unless given), Q, K pool, V pool, new K, new V.
    ``order`` is "round_robin" (token j of the ubatch belongs to the next sequence
    that still has tokens, cycling) or "grouped" (each sequence's tokens together).
    """
    if perm is None:
        perm = rng.permutation(num_pages)
    prefixes = np.asarray(prefixes, dtype=np.int64)
    n_new = np.asarray(n_new, dtype=np.int64)
    totals = prefixes + n_new
    bt, valid_total = _assign_pages(perm, totals, page_size)
    # token order
    toks = []  # (seq, pos)
    if order == "grouped":
        for s in range(len(prefixes)):
            toks += [(s, int(prefixes[s] + j)) for j in range(int(n_new[s]))]
    elif order == "round_robin":
        left = [int(x) for x in n_new]
        done = [0] * len(left)
        while sum(left) > 0:
            for s in range(len(left)):
                if left[s] > 0:
                    toks.append((s, int(prefixes[s] + done[s])))
                    done[s] += 1
                    left[s] -= 1
    else:
        raise ValueError(order)
    T = len(toks)
    token_row = np.array([t[0] for t in toks], dtype=np.int32)
    token_pos = np.array([t[1] for t in toks], dtype=np.int32)
    token_kv_len = totals[token_row].astype(np.int32)
    slot = np.empty(T, dtype=np.int32)
    valid_prefix = np.zeros_like(valid_total)
    for s in range(len(prefixes)):
        for j in range(int(prefixes[s])):
            page = bt[s, j // page_size]
            valid_prefix[page, j % page_size] = True
    for i, (s, pos) in enumerate(toks):
        slot[i] = bt[s, pos // page_size] * page_size + pos % page_size
    q = _normal(rng, (T, n_q_heads, head_dim), std)
    k, v = _draw_pools(rng, num_pages, n_kv_heads, page_size, head_dim, std)
    poison_pools(k, v, valid_prefix)
    k_new = _normal_f16(rng, (T, n_kv_heads, head_dim), std)
    v_new = _normal_f16(rng, (T, n_kv_heads, head_dim), std)
    return PrefillCase(name, n_q_heads, n_kv_heads, head_dim, page_size, num_pages, q, k, v,
                       k_new, v_new, slot, bt, token_row, token_kv_len, token_pos,
                       fp32_scale(head_dim), totals.astype(np.int32))


def ua_prefill(n_seqs=8, new_per_seq=64, lo=2048, hi=16384, num_pages=2048) -> PrefillCase:
    """512 query tokens interleaved round-robin from 8 sequences (64 new each),
    appended after prefixes drawn uniformly from {2048..16384}; GQA 32/8, D 128, P 128."""
    rng = rng_for(2)
    perm = rng.permutation(num_pages)
    prefixes = rng.integers(lo, hi + 1, size=n_seqs)
    return make_prefill_case(rng, f"ua_prefill_{n_seqs}x{new_per_seq}_prefix{lo}-{hi}", 32, 8, 128,
                             128, num_pages, prefixes, [new_per_seq] * n_seqs, "round_robin",
                             1.0, perm)


@dataclass
class ChunkedPrefill:
    """Fresh sequences prefilled in fixed-size ubatches, one sequence per ubatch,
    chunk-major order (chunk outer, sequence inner)."""
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    chunk: int
    seq_len: int
    free_order: np.ndarray     # int32 [N] page hand-out order for the pool
    q: np.ndarray              # float32 [S][L][Hq][D]
    k: np.ndarray              # float16 [S][L][Hkv][D]
    v: np.ndarray              # float16 [S][L][Hkv][D]
    scale: np.float32

    @property
    def n_seqs(self):
        return self.q.shape[0]

    def ubatches(self):
        """Yield (seq, first_pos) for every ubatch in execution order."""
        for c in range(self.seq_len // self.chunk):
            for s in range(self.n_seqs):
                yield s, c * self.chunk


def chunked_prefill(n_seqs=8, seq_len=16384, chunk=512, num_pages=2048, config_index=4,
                    rng=None) -> ChunkedPrefill:
    """8 fresh sequences x 16384 tokens in 512-token ubatches; GQA 32/8, D 128, P 128,
    values N(0,1).  Draw order: free-page order, Q, K, V."""
    rng = rng_for(config_index) if rng is None else rng
    free_order = rng.permutation(num_pages).astype(np.int32)
    q = _normal(rng, (n_seqs, seq_len, 32, 128))
    k = _normal_f16(rng, (n_seqs, seq_len, 8, 128))
    v = _normal_f16(rng, (n_seqs, seq_len, 8, 128))
    return ChunkedPrefill(32, 8, 128, 128, num_pages, chunk, seq_len, free_order, q, k, v,
                          fp32_scale(128))


@dataclass
class SharingCase:
    """A refcounted shared prefix with private suffixes (copy-on-write workload).

    Sequence 0 is created and filled with the prefix, then forked ``n_seqs-1``
    times; every sequence then appends its private suffix; one decode query per
    sequence.
    """
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    free_order: np.ndarray       # int32 [N]
    prefix_k: np.ndarray         # float16 [Lp][Hkv][D]
    prefix_v: np.ndarray
    suffix_k: np.ndarray         # float16 [S][Ls][Hkv][D]
    suffix_v: np.ndarray
    q: np.ndarray                # float32 [S][Hq][D]
    scale: np.float32


def sharing_case(n_seqs=16, prefix_len=8192, suffix_len=1024, page_size=128, num_pages=2048,
                 n_q_heads=32, n_kv_heads=8, head_dim=128, config_index=4) -> SharingCase:
    """16 sequences sharing an 8192-token prefix, each with a private 1024-token
    suffix; GQA 32/8, D 128, P 128, N(0,1).  Draw order: free-page order, Q, K, V."""
    rng = rng_for(config_index)
    free_order = rng.permutation(num_pages).astype(np.int32)
    q = _normal(rng, (n_seqs, n_q_heads, head_dim))
    pk = _normal_f16(rng, (prefix_len, n_kv_heads, head_dim))
    sk = _normal_f16(rng, (n_seqs, suffix_len, n_kv_heads, head_dim))
    pv = _normal_f16(rng, (prefix_len, n_kv_heads, head_dim))
    sv = _normal_f16(rng, (n_seqs, suffix_len, n_kv_heads, head_dim))
    return SharingCase(n_q_heads, n_kv_heads, head_dim, page_size, num_pages, free_order,
                       pk, pv, sk, sv, q, fp32_scale(head_dim))


def nan_pools(num_pages, n_kv_heads, page_size, head_dim):
    """An all-NaN (empty) pool pair."""
    ks, vs = _pool_shapes(num_pages, n_kv_heads, page_size, head_dim)
    k = np.empty(ks, dtype=np.float16)
    v = np.empty(vs, dtype=np.float16)
    k.view(np.uint16)[...] = NAN_F16_BITS
    v.view(np.uint16)[...] = NAN_F16_BITS
    return k, v


__all__.append("nan_pools")


# ---------------------------------------------------------------- work counts

def decode_valid_bytes(kv_lens, n_kv_heads, head_dim, elem_bytes=2) -> int:
    """Bytes of valid K and V a decode pass must read: every valid cell once."""
    return int(np.sum(np.asarray(kv_lens, dtype=np.int64))) * n_kv_heads * head_dim * elem_bytes * 2


def prefill_pairs(token_kv_len, token_pos, token_row=None) -> int:
    """Number of (query token, key) pairs a prefill attends: sum of min(kv_len, pos+1)."""
    n = np.minimum(np.asarray(token_kv_len, np.int64), np.asarray(token_pos, np.int64) + 1)
    if token_row is not None:
        n = np.where(np.asarray(token_row) >= 0, n, 0)
    return int(n.sum())


def attention_flops(pairs: int, n_q_heads: int, head_dim: int) -> int:
    """QK^T and PV at 2 flop per multiply-add: 4 * D * Hq per attended pair."""
    return 4 * head_dim * n_q_heads * int(pairs)


# ---------------------------------------------------------------- unified span

def unified_view(block_tables, seq_lens, num_pages, page_size):
    """The unified-cache view of a paged pool: the span is cells 0..span-1 of the
    pool read as one flat array (cell c = page c // P, slot c % P), covering every
    page any sequence uses; ``cell_seq[c]`` / ``cell_pos[c]`` say which sequence
    position the cell holds (-1 / 0 for free cells and the unused tail of a
    sequence's last page).  ``seq_lens[r]`` is the number of cells row r of
    ``block_tables`` holds.  Returns (span, cell_seq int32 [span], cell_pos int32
    [span]); the span is rounded up to a whole page."""
    bt = np.asarray(block_tables)
    cell_seq = np.full(num_pages * page_size, -1, dtype=np.int32)
    cell_pos = np.zeros(num_pages * page_size, dtype=np.int32)
    last = -1
    for r, n in enumerate(np.asarray(seq_lens, dtype=np.int64)):
        t = np.arange(int(n))
        pages = bt[r, t // page_size].astype(np.int64)
        cells = pages * page_size + t % page_size
        cell_seq[cells] = r
        cell_pos[cells] = t
        if n > 0:
            last = max(last, int(pages.max()))
    span = (last + 1) * page_size
    return span, cell_seq[:span].copy(), cell_pos[:span].copy()


def unified_decode_bytes(span, n_kv_heads, head_dim, elem_bytes=2) -> int:
    """Bytes of K and V a unified-span pass reads: every cell of the span once."""
    return int(span) * n_kv_heads * head_dim * elem_bytes * 2


def unified_pairs(span, n_tokens_real) -> int:
    """(query token, cell) pairs a unified-span pass computes: every real token
    against every cell of the span (the mask removes most of them from the
    result, not from the work)."""
    return int(span) * int(n_tokens_real)


__all__ += ["unified_view", "unified_decode_bytes", "unified_pairs"]


# ---------------------------------------------------------------- token-keyed K/V

@dataclass
class TokenKV:
    """A seeded stand-in for a model's K/V projections in which a token's K and V
    depend only on its id and its position: two requests whose leading tokens are
    equal then hold equal K/V there, which is what lets one reuse the other's
    cached pages.  Tables are float32; ``kv`` rounds their sum to float16."""
    ek: np.ndarray      # float32 [vocab][Hkv][D]
    ev: np.ndarray
    pk: np.ndarray      # float32 [max_pos][Hkv][D]
    pv: np.ndarray

    def kv(self, tokens, positions):
        t = np.asarray(tokens, dtype=np.int64)
        p = np.asarray(positions, dtype=np.int64)
        k = (self.ek[t] + self.pk[p]).astype(np.float16)
        v = (self.ev[t] + self.pv[p]).astype(np.float16)
        return k, v


def token_kv(seed, vocab, max_pos, n_kv_heads=8, head_dim=128) -> TokenKV:
    """Draw order: token K, token V, position K, position V; N(0,1)*0.8 for the
    token part and N(0,1)*0.6 for the position part (unit variance overall)."""
    rng = np.random.default_rng(seed)
    ek = _normal(rng, (vocab, n_kv_heads, head_dim), 0.8)
    ev = _normal(rng, (vocab, n_kv_heads, head_dim), 0.8)
    pk = _normal(rng, (max_pos, n_kv_heads, head_dim), 0.6)
    pv = _normal(rng, (max_pos, n_kv_heads, head_dim), 0.6)
    return TokenKV(ek, ev, pk, pv)


__all__ += ["TokenKV", "token_kv"]
