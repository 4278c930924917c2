"""Prefix cache on the GPU: requests that reuse a cached prefix through
pa_prefix_match read the first request's physical pages, prefill only their own
tokens, and get exactly the attention outputs (bit for bit) that the same
ubatches give on a private pool where every request holds its own copy, within
tolerance of the oracle over each request's logical K/V; after eviction and
after compaction the reused pages still hold the right K/V."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_185_amd as pa
import workloads as W
from gpu_util import assert_attention_close, bits16, to_dev, to_host

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128
SCALE = W.fp32_scale(D)


def requests(rng, vocab=500):
    system = list(rng.integers(0, vocab, 600))
    return [system + list(rng.integers(0, vocab, 100)),        # A: first, inserted
            system + list(rng.integers(0, vocab, 150)),        # B: whole system prompt
            system[:300] + list(rng.integers(0, vocab, 50)),   # C: part of it
            list(rng.integers(0, vocab, 80))]                  # D: nothing shared


class Server:
    """Admits requests into one paged pool and runs prefill / decode ubatches."""

    def __init__(self, num_pages, P, tkv, seed):
        self.P = P
        self.tkv = tkv
        self.pool = pa.Pool(num_pages, P, np.random.default_rng(seed).permutation(num_pages))
        k, v = W.nan_pools(num_pages, HKV, P, D)
        self.kd, self.vd = to_dev(k), to_dev(v)
        self.seq = {}
        self.toks = {}

    def write(self, r, toks, start):
        """Appends toks[start:] to request r's sequence and caches their K/V."""
        slots, cow = self.pool.seq_append(self.seq[r], len(toks) - start)
        assert cow is None
        if len(slots):
            k, v = self.tkv.kv(toks[start:], np.arange(start, len(toks)))
            pa.pa_reshape_and_cache(self.kd, self.vd, to_dev(k), to_dev(v), to_dev(slots))
        self.toks[r] = list(toks)

    def admit(self, reqs, batch, qtab, use_prefix, starts=None):
        """Creates sequences for `batch`, writes their K/V and prefills one
        ubatch holding, for each request, the queries from its start position
        (the matched length, or the given one) to its end."""
        got = {}
        for r in batch:
            toks = reqs[r]
            if use_prefix:
                s, m = self.pool.prefix_match(toks)
            else:
                s, m = self.pool.seq_new(), 0
            self.seq[r] = s
            self.write(r, toks, m)
            got[r] = m if starts is None else starts[r]
        return got, self.prefill(batch, got, qtab)

    def table(self, batch):
        mp = max(len(self.toks[r]) for r in batch) // self.P + 1
        bt, kv = self.pool.block_tables([self.seq[r] for r in batch], mp)
        return bt, kv

    def prefill(self, batch, starts, qtab):
        bt, kv = self.table(batch)
        row, kvl, pos, q = [], [], [], []
        for i, r in enumerate(batch):
            n = len(self.toks[r])
            for p in range(starts[r], n):
                row.append(i)
                kvl.append(n)
                pos.append(p)
                q.append(qtab[r][p])
        row, kvl, pos = (np.asarray(x, dtype=np.int32) for x in (row, kvl, pos))
        q = np.stack(q).astype(np.float32)
        out = pa.pa_prefill(to_dev(q), self.kd, self.vd, to_dev(bt), to_dev(row), to_dev(kvl),
                            to_dev(pos), float(SCALE), token_row_host=row, token_kv_len_host=kvl,
                            token_pos_host=pos)
        return dict(q=q, row=row, kvl=kvl, pos=pos, out=to_host(out))

    def decode(self, batch, new_tok, qdec):
        for r in batch:
            self.write(r, self.toks[r] + [new_tok[r]], len(self.toks[r]))
        bt, kv = self.table(batch)
        out = pa.pa_decode(to_dev(qdec), self.kd, self.vd, to_dev(bt), to_dev(kv), float(SCALE),
                           kv_lens_host=kv)
        return kv, to_host(out)


def logical_pools(tkv, toks_list, P):
    """Each request's K/V from its tokens alone, in private pages 0.. of a host
    pool, with the identity block table (the oracle's view).  V is filled as
    value columns [N][Hkv][D][P] and returned in V storage order."""
    n_pages = [-(-len(t) // P) for t in toks_list]
    N = sum(n_pages)
    k = np.zeros((N, HKV, P, D), np.float16)
    v = np.zeros((N, HKV, D, P), np.float16)
    bt = np.full((len(toks_list), max(n_pages)), -1, np.int32)
    base = 0
    for i, t in enumerate(toks_list):
        kk, vv = tkv.kv(t, np.arange(len(t)))
        for j in range(n_pages[i]):
            c = kk[j * P:(j + 1) * P]
            k[base + j, :, :len(c)] = c.transpose(1, 0, 2)
            v[base + j, :, :, :len(c)] = vv[j * P:(j + 1) * P].transpose(1, 2, 0)
            bt[i, j] = base + j
        base += n_pages[i]
    return k, W.v_blocks_from_columns(v), bt


@pytest.mark.parametrize("P", [16, 128])
def test_prefix_reuse_is_bitwise_equal_to_private_pages(P):
    rng = np.random.default_rng(80 + P)
    reqs = requests(rng)
    tkv = W.token_kv(81, 500, 1024, HKV, D)
    qtab = [rng.standard_normal((len(t) + 1, HQ, D), dtype=np.float32) for t in reqs]
    new_tok = [int(x) for x in rng.integers(0, 500, 4)]
    qdec = np.stack([qtab[r][len(reqs[r])] for r in range(4)])
    N = 2048 // P

    shared = Server(N, P, tkv, seed=1)
    _, first_s = shared.admit(reqs, [0], qtab, use_prefix=True)
    assert shared.pool.prefix_insert(shared.seq[0], reqs[0]) == len(reqs[0]) // P
    starts, second_s = shared.admit(reqs, [1, 2, 3], qtab, use_prefix=True)
    assert starts == {1: 600 // P * P, 2: 300 // P * P, 3: 0}
    bt, _ = shared.table([0, 1, 2, 3])
    n_sys, n_half = 600 // P, 300 // P
    assert np.array_equal(bt[1, :n_sys], bt[0, :n_sys])          # the same physical pages
    assert np.array_equal(bt[2, :n_half], bt[0, :n_half])
    _, ref = shared.pool.stats()
    assert np.all(ref[bt[0, :n_half]] == 4) and np.all(ref[bt[0, n_half:n_sys]] == 3)
    kv_s, dec_s = shared.decode([0, 1, 2, 3], new_tok, qdec)

    private = Server(N, P, tkv, seed=2)
    _, first_p = private.admit(reqs, [0], qtab, use_prefix=False)
    _, second_p = private.admit(reqs, [1, 2, 3], qtab, use_prefix=False, starts=starts)
    kv_p, dec_p = private.decode([0, 1, 2, 3], new_tok, qdec)
    used_s = N - shared.pool.stats()[0]
    used_p = N - private.pool.stats()[0]
    assert used_p - used_s == n_sys + n_half                     # pages the cache saved

    assert np.array_equal(first_s["out"].view(np.uint32), first_p["out"].view(np.uint32))
    assert np.array_equal(second_s["out"].view(np.uint32), second_p["out"].view(np.uint32))
    assert np.array_equal(kv_s, kv_p)
    assert np.array_equal(dec_s.view(np.uint32), dec_p.view(np.uint32))

    # oracle over each request's own K/V
    full = [reqs[r] + [new_tok[r]] for r in range(4)]
    k, v, lbt = logical_pools(tkv, full, P)
    rows = np.array([1, 2, 3])[second_s["row"]]
    ref2 = oracle.paged_attention(second_s["q"], k, v, lbt, rows, second_s["kvl"], second_s["pos"],
                                  SCALE)
    assert_attention_close(second_s["out"], ref2, f"prefill after prefix match, P={P}")
    ref3 = oracle.paged_decode(qdec, k, v, lbt, kv_s, SCALE)
    assert_attention_close(dec_s, ref3, f"decode on shared pages, P={P}")


def test_evicted_pages_are_reused_cleanly():
    """A pool too small for a new request until the cache gives pages back: the
    evicted pages are rewritten and the new request's attention is exact."""
    P = 16
    rng = np.random.default_rng(90)
    tkv = W.token_kv(91, 300, 512, HKV, D)
    a = list(rng.integers(0, 300, 320))            # 20 pages
    b = list(rng.integers(0, 300, 400))            # 25 pages, shares nothing with a
    N = 32
    srv = Server(N, P, tkv, seed=3)
    qtab = [rng.standard_normal((len(t), HQ, D), dtype=np.float32) for t in (a, b)]
    srv.admit([a, b], [0], qtab, use_prefix=True)
    srv.pool.prefix_insert(srv.seq[0], a)
    srv.pool.seq_free(srv.seq[0])
    assert srv.pool.stats()[0] == N - 20 and srv.pool.prefix_pages() == 20
    s, m = srv.pool.prefix_match(b)
    assert m == 0
    with pytest.raises(pa.NoPagesError):
        srv.pool.seq_append(s, len(b))
    assert srv.pool.prefix_evict(25 - (N - 20)) == 13
    srv.pool.seq_free(s)
    _, res = srv.admit([a, b], [1], qtab, use_prefix=True)
    k, v, lbt = logical_pools(tkv, [b], P)
    ref = oracle.paged_attention(res["q"], k, v, lbt, res["row"], res["kvl"], res["pos"], SCALE)
    assert_attention_close(res["out"], ref, "prefill on evicted pages")


def test_compaction_moves_cached_pages_and_matches_still_read_them():
    """Cached pages above n_live are moved by pa_pool_compact + pa_copy_blocks;
    a later match receives the moved pages, whose bytes equal the originals."""
    P = 16
    rng = np.random.default_rng(95)
    tkv = W.token_kv(96, 300, 512, HKV, D)
    reqs = [list(rng.integers(0, 300, n)) for n in (200, 240, 160)]
    qtab = [rng.standard_normal((len(t) + 1, HQ, D), dtype=np.float32) for t in reqs]
    N = 64
    srv = Server(N, P, tkv, seed=4)
    srv.admit(reqs, [0, 1, 2], qtab, use_prefix=True)
    srv.pool.prefix_insert(srv.seq[1], reqs[1])
    before = bits16(to_host(srv.kd)).copy(), bits16(to_host(srv.vd)).copy()
    bt1, _ = srv.table([1])
    cached = bt1[0, :len(reqs[1]) // P].copy()
    srv.pool.seq_free(srv.seq[0])
    srv.pool.seq_free(srv.seq[1])
    pairs = srv.pool.compact()
    assert len(pairs)
    pa.pa_copy_blocks([srv.kd], [srv.vd], pairs)
    moved = dict((int(s), int(d)) for s, d in pairs)
    s, m = srv.pool.prefix_match(reqs[1] + [1, 2, 3])
    assert m == len(reqs[1]) // P * P
    got_pages = srv.pool.block_tables([s], m // P)[0][0]
    assert list(got_pages) == [moved.get(int(p), int(p)) for p in cached]
    kd, vd = bits16(to_host(srv.kd)), bits16(to_host(srv.vd))
    for p_old, p_new in zip(cached, got_pages):
        assert np.array_equal(kd[p_new], before[0][p_old])
        assert np.array_equal(vd[p_new], before[1][p_old])
    srv.seq[1] = s
    srv.toks[1] = reqs[1][:m]
    qdec = qtab[1][m][None]
    kv, out = srv.decode([1], {1: 7}, qdec)
    k, v, lbt = logical_pools(tkv, [reqs[1][:m] + [7]], P)
    ref = oracle.paged_decode(qdec, k, v, lbt, kv, SCALE)
    assert_attention_close(out, ref, "decode on compacted cached pages")
