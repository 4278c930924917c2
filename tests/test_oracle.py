"""Pins for the CPU oracle (no GPU).

The pages print no worked example, so each oracle function is pinned to
something other than itself: a pure-Python brute force that walks the physical
pool through inverted block tables, torch's float64 CPU attention on inputs
that need no paging, hand-derived fixtures, closed forms and invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from pool_script import run_pool_script

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- brute force

def vcol(v_pool, page, h, slot):
    """Value column of (page, KV head h, slot) read from V storage
    [N][Hkv][P // B][D][B], B = min(P, 32), written out independently of the
    oracle's gather."""
    P = v_pool.shape[2] * v_pool.shape[4]
    B = min(P, 32)
    assert v_pool.shape[4] == B
    return v_pool[page, h, slot // B, :, slot % B]


def vcols(v_pool):
    """V storage [N][Hkv][P // B][D][B] as value columns [N][Hkv][D][P] (a copy)."""
    N, H, nb, D, B = v_pool.shape
    return v_pool.transpose(0, 1, 3, 2, 4).reshape(N, H, D, nb * B)


def brute_force(q, k_pool, v_pool, block_tables, token_row, token_kv_len, token_pos, scale):
    """Scalar definition.  Inverts the block tables (physical cell -> (row, logical
    position)) instead of gathering, then loops with math.fsum / math.exp."""
    _, n_kv, P, D = k_pool.shape
    T, n_q, _ = q.shape
    G = n_q // n_kv
    owner = {}
    for r, row in enumerate(np.asarray(block_tables)):
        for j, page in enumerate(row):
            if page >= 0:
                for s in range(P):
                    owner.setdefault((int(page), s), []).append((r, j * P + s))
    sc = float(np.float32(scale))
    out = np.zeros((T, n_q, D))
    for i in range(T):
        r = int(token_row[i])
        if r < 0:
            continue
        n = min(int(token_kv_len[i]), int(token_pos[i]) + 1)
        cells = sorted((t, page, s) for (page, s), lst in owner.items()
                       for (rr, t) in lst if rr == r and t < n)
        assert [c[0] for c in cells] == list(range(n))
        for h in range(n_q):
            g = h // G
            qv = [float(x) for x in q[i, h]]
            z = [sc * math.fsum(qv[d] * float(k_pool[p, g, s, d]) for d in range(D))
                 for (_, p, s) in cells]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            den = math.fsum(w)
            for d in range(D):
                out[i, h, d] = math.fsum(w[c] * float(vcol(v_pool, cells[c][1], g, cells[c][2])[d])
                                         for c in range(n)) / den
    return out


def _small_prefill(seed=7, order="round_robin"):
    rng = np.random.default_rng(seed)
    case = W.make_prefill_case(rng, "small", 4, 2, 32, 16, 24, [20, 33, 5], [6, 4, 7], order)
    k, v = oracle.reshape_and_cache(case.k_pool, case.v_pool, case.k_new, case.v_new,
                                    case.slot_mapping)
    return case, k, v


def test_brute_force_tiny_decode():
    c = W.tiny_decode()
    got = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    ref = brute_force(c.q, c.k_pool, c.v_pool, c.block_tables, np.arange(2), c.kv_lens,
                      c.kv_lens - 1, c.scale)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("order", ["round_robin", "grouped"])
def test_brute_force_small_prefill(order):
    c, k, v = _small_prefill(order=order)
    got = oracle.paged_attention(c.q, k, v, c.block_tables, c.token_row, c.token_kv_len,
                                 c.token_pos, c.scale)
    ref = brute_force(c.q, k, v, c.block_tables, c.token_row, c.token_kv_len, c.token_pos,
                      c.scale)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("P", [64, 128])
def test_brute_force_multi_block_v_pages(P):
    """Pages of more than one V slot block (P > 32), with ragged last pages and
    NaN in their unused cells: the oracle's gather of blocked V storage against
    the brute force's own cell-by-cell reading."""
    rng = np.random.default_rng(12 + P)
    c = W.make_decode_case(rng, "blocks", 4, 2, 8, P, [P + 37, 2 * P - 5, 33], 9)
    got = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    ref = brute_force(c.q, c.k_pool, c.v_pool, c.block_tables, np.arange(3), c.kv_lens,
                      c.kv_lens - 1, c.scale)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_reshape_then_gather_round_trip_multi_block():
    """Tokens scattered by reshape_and_cache into 128-slot pages come back in
    order from the oracle's gather (both read the blocked V storage, each in
    its own code), and the V cell of slot s holds token s's value column."""
    rng = np.random.default_rng(13)
    N, Hkv, P, D = 5, 2, 128, 8
    k, v = W.nan_pools(N, Hkv, P, D)
    T = 300
    kn = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    pages = np.array([3, 0, 4])
    slots = (pages[np.arange(T) // P] * P + np.arange(T) % P).astype(np.int32)
    k2, v2 = oracle.reshape_and_cache(k, v, kn, vn, slots)
    K, V = oracle.gather_logical(k2, v2, pages, T)
    np.testing.assert_array_equal(K, kn.astype(np.float64))
    np.testing.assert_array_equal(V, vn.astype(np.float64))
    for t in (0, 31, 32, 63, 64, 127, 128, 200, 299):
        for h in range(Hkv):
            np.testing.assert_array_equal(vcol(v2, pages[t // P], h, t % P), vn[t, h])


def test_brute_force_shared_pages():
    """Two rows whose tables share their first page (a forked prefix)."""
    rng = np.random.default_rng(11)
    N, Hkv, P, D = 8, 1, 4, 16
    k = rng.standard_normal((N, Hkv, P, D)).astype(np.float16)
    v = W.v_blocks_from_columns(rng.standard_normal((N, Hkv, D, P)).astype(np.float16))
    bt = np.array([[6, 1, -1], [6, 3, 0]], dtype=np.int32)
    q = rng.standard_normal((2, 2, D)).astype(np.float32)
    lens = np.array([7, 10], dtype=np.int32)
    got = oracle.paged_decode(q, k, v, bt, lens, 0.25)
    ref = brute_force(q, k, v, bt, np.arange(2), lens, lens - 1, 0.25)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ golden fixtures

def _hand_pool(g):
    pool = g["pool"]
    k, v = W.nan_pools(pool["num_pages"], pool["n_kv_heads"], pool["page_size"], pool["head_dim"])
    for c in pool["cells"]:
        for h in range(pool["n_kv_heads"]):
            k[c["page"], h, c["slot"], :] = c["k"][h]
            vcol(v, c["page"], h, c["slot"])[:] = c["v"][h]
    return k, v, np.array(pool["block_table"], dtype=np.int32)


def test_golden_attention_hand():
    g = json.load(open(os.path.join(GOLD, "attention_hand.json")))
    k, v, bt = _hand_pool(g)
    for case in g["cases"]:
        T = len(case["token_row"])
        q = np.array([g["queries"]] * T, dtype=np.float32)
        got = oracle.paged_attention(q, k, v, bt, case["token_row"], case["token_kv_len"],
                                     case["token_pos"], g["scale"])
        np.testing.assert_allclose(got, np.array(case["expected"], dtype=np.float64),
                                   rtol=1e-15, atol=1e-15, err_msg=case["name"])


# ------------------------------------------------------- torch float64 SDPA

def _sdpa(q, K, V, G, scale, mask):
    """q [T][Hq][D], K/V [n][Hkv][D] float64; mask bool [T][n] (True = visible)."""
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=float(np.float32(scale)))
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv,D,L", [(4, 2, 64, 37), (8, 8, 32, 16), (32, 8, 128, 100)])
def test_sdpa_single_page(Hq, Hkv, D, L):
    """One sequence in one page (P >= L): no paging, so torch's attention applies."""
    rng = np.random.default_rng(L)
    P = 128
    k = rng.standard_normal((3, Hkv, P, D)).astype(np.float16)
    v_cols = rng.standard_normal((3, Hkv, D, P)).astype(np.float16)   # value columns per slot
    v = W.v_blocks_from_columns(v_cols)
    bt = np.array([[2]], dtype=np.int32)
    T = 5
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    pos = np.array([L - 1, L - 2, 0, L - 5, L - 1], dtype=np.int32)
    got = oracle.paged_attention(q, k, v, bt, np.zeros(T, np.int32), np.full(T, L, np.int32),
                                 pos, 1.0 / math.sqrt(D))
    K = k[2, :, :L, :].transpose(1, 0, 2).astype(np.float64)
    V = v_cols[2, :, :, :L].transpose(2, 0, 1).astype(np.float64)
    mask = np.arange(L)[None, :] <= pos[:, None]
    ref = _sdpa(q, K, V, Hq // Hkv, 1.0 / math.sqrt(D), mask)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms

def _one_seq(rng, L, Hq=4, Hkv=2, D=16, P=8, N=12):
    case = W.make_decode_case(rng, "cf", Hq, Hkv, D, P, [L], N)
    return case


def test_closed_form_single_key():
    c = _one_seq(np.random.default_rng(1), 1)
    out = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    page = c.block_tables[0, 0]
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], vcol(c.v_pool, page, h // 2, 0).astype(np.float64))


def test_closed_form_zero_query_is_mean():
    c = _one_seq(np.random.default_rng(2), 29)
    q = np.zeros_like(c.q)
    out = oracle.paged_decode(q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    # independent computation of the mean from the physical pool
    P = 8
    vals = np.stack([[vcol(c.v_pool, c.block_tables[0, t // P], g, t % P) for g in range(2)]
                     for t in range(29)])
    for h in range(4):
        np.testing.assert_allclose(out[0, h], vals[:, h // 2, :].astype(np.float64).mean(0),
                                   rtol=1e-13, atol=1e-14)


def test_closed_form_identical_keys_is_mean_and_constant_v():
    rng = np.random.default_rng(3)
    c = _one_seq(rng, 21)
    valid = c.valid_cells
    k = c.k_pool.copy()
    # every valid cell of KV head g gets the same key row
    for g in range(2):
        row = rng.standard_normal(16).astype(np.float16)
        kg = k[:, g]                                        # [N][P][D]
        kg[valid] = row
    out = oracle.paged_decode(c.q, k, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    vals = np.stack([[vcol(c.v_pool, c.block_tables[0, t // 8], g, t % 8) for g in range(2)]
                     for t in range(21)])
    for h in range(4):
        np.testing.assert_allclose(out[0, h], vals[:, h // 2].astype(np.float64).mean(0),
                                   rtol=1e-13, atol=1e-14)
    # constant V (value depends on the KV head) -> that constant, whatever the keys
    v = c.v_pool.copy()
    for g in range(2):
        for page, slot in zip(*np.nonzero(valid)):
            vcol(v, page, g, slot)[:] = np.float16(0.5 * (g + 1))
    out = oracle.paged_decode(c.q, c.k_pool, v, c.block_tables, c.kv_lens, c.scale)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], 0.5 * (h // 2 + 1), rtol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(4)
    c = W.make_decode_case(rng, "g", 8, 2, 16, 8, [13, 30], 16)
    out = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    G = 4
    k_rep = np.repeat(c.k_pool, G, axis=1)
    v_rep = np.repeat(c.v_pool, G, axis=1)
    out_mha = oracle.paged_decode(c.q, k_rep, v_rep, c.block_tables, c.kv_lens, c.scale)
    # BLAS may block a 4-row product differently from 1-row products: rounding only
    np.testing.assert_allclose(out, out_mha, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ invariants

def test_page_permutation_bitwise():
    c = W.tiny_decode()
    out = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    pi = np.random.default_rng(5).permutation(c.num_pages)   # old page p -> new id pi[p]
    k2 = np.empty_like(c.k_pool)
    v2 = np.empty_like(c.v_pool)
    k2[pi] = c.k_pool
    v2[pi] = c.v_pool
    bt2 = np.where(c.block_tables >= 0, pi[np.maximum(c.block_tables, 0)], -1)
    out2 = oracle.paged_decode(c.q, k2, v2, bt2, c.kv_lens, c.scale)
    np.testing.assert_array_equal(out, out2)


def test_nan_poison_does_not_change_output():
    c = W.tiny_decode()
    out = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    assert np.all(np.isfinite(out))
    # replace every poisoned cell by finite garbage; the output must not move
    rng = np.random.default_rng(6)
    k = c.k_pool.copy()
    v = c.v_pool.copy()
    k[np.isnan(k)] = rng.standard_normal(int(np.isnan(k).sum())).astype(np.float16) * 100
    v[np.isnan(v)] = rng.standard_normal(int(np.isnan(v).sum())).astype(np.float16) * 100
    out2 = oracle.paged_decode(c.q, k, v, c.block_tables, c.kv_lens, c.scale)
    np.testing.assert_array_equal(out, out2)
    # and the poisoned case really is poisoned: free pages and padding are NaN
    n_nan_pages = int(np.all(np.isnan(c.k_pool.reshape(c.num_pages, -1)), axis=1).sum())
    assert n_nan_pages == c.num_pages - 16


@pytest.mark.parametrize("part", [16, 32, 48, 64, 200, 1000])
def test_lse_split_identity(part):
    c = W.tiny_decode()
    out = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    out2, m, l, acc = oracle.partitioned_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                                c.kv_lens, c.scale, part)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    n_part = m.shape[-1]
    assert n_part == max(1, -(-200 // part))
    # partitions beyond sequence 0's length are empty
    used0 = -(-37 // part)
    assert np.all(np.isneginf(m[0, :, used0:])) and np.all(l[0, :, used0:] == 0)


def test_decode_is_ua_special_case():
    c = W.tiny_decode()
    a = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    # the same two queries presented as a ubatch in reverse order with a padding token
    q = np.stack([c.q[1], np.zeros_like(c.q[0]), c.q[0]])
    b = oracle.paged_attention(q, c.k_pool, c.v_pool, c.block_tables, [1, -1, 0],
                               [200, 0, 37], [199, 0, 36], c.scale)
    np.testing.assert_array_equal(b[0], a[1])
    np.testing.assert_array_equal(b[2], a[0])
    assert np.all(b[1] == 0)


def test_oracle_reads_only_needed_pages():
    """Pages past ceil(n/P) may be garbage ids; the oracle must not touch them."""
    c = W.tiny_decode()
    bt = c.block_tables.copy()
    bt[0, 3:] = 10 ** 6
    a = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    b = oracle.paged_decode(c.q, c.k_pool, c.v_pool, bt, c.kv_lens, c.scale)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------- cache ops

def test_f16_rounding_golden():
    g = json.load(open(os.path.join(GOLD, "f16_rounding.json")))
    bits = np.array([int(c[0], 16) for c in g["cases"]], dtype=np.uint32)
    want = np.array([int(c[1], 16) for c in g["cases"]], dtype=np.uint16)
    n = len(bits)
    src = np.zeros((n, 1, 1), dtype=np.float32)
    src[:, 0, 0] = bits.view(np.float32)
    k, v = W.nan_pools(n, 1, 1, 1)
    with np.errstate(over="ignore"):
        k2, v2 = oracle.reshape_and_cache(k, v, src, src, np.arange(n, dtype=np.int32))
    np.testing.assert_array_equal(k2.view(np.uint16).ravel(), want)
    np.testing.assert_array_equal(v2.view(np.uint16).ravel(), want)
    nb = np.array([int(x, 16) for x in g["nan"]], dtype=np.uint32).view(np.float32)
    k, v = W.nan_pools(len(nb), 1, 1, 1)
    k.view(np.uint16)[...] = 0
    k3, _ = oracle.reshape_and_cache(k, v, nb.reshape(-1, 1, 1), nb.reshape(-1, 1, 1),
                                     np.arange(len(nb), dtype=np.int32))
    assert np.all(np.isnan(k3))


def test_reshape_and_cache_touches_only_addressed_cells():
    rng = np.random.default_rng(8)
    N, Hkv, P, D = 10, 3, 8, 16
    k = rng.standard_normal((N, Hkv, P, D)).astype(np.float16)
    v = W.v_blocks_from_columns(rng.standard_normal((N, Hkv, D, P)).astype(np.float16))
    T = 7
    kn = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    slots = np.array([3, 17, -1, 79, 40, -5, 8], dtype=np.int32)
    k2, v2 = oracle.reshape_and_cache(k, v, kn, vn, slots)
    kb, k2b = k.view(np.uint16), k2.view(np.uint16)
    vb, v2b = vcols(v).view(np.uint16), vcols(v2).view(np.uint16)
    touched = np.zeros((N, P), dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        p, o = divmod(int(s), P)
        touched[p, o] = True
        for h in range(Hkv):
            for d in range(D):
                assert k2b[p, h, o, d] == kn[i, h, d].view(np.uint16)
                assert v2b[p, h, d, o] == vn[i, h, d].view(np.uint16)
    for p in range(N):
        for o in range(P):
            if not touched[p, o]:
                assert np.array_equal(k2b[p, :, o, :], kb[p, :, o, :])
                assert np.array_equal(v2b[p, :, :, o], vb[p, :, :, o])
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(k, v, kn[:2], vn[:2], np.array([5, 5], np.int32))


def test_copy_blocks():
    rng = np.random.default_rng(9)
    N = 9
    ks = [rng.standard_normal((N, 2, 4, 8)).astype(np.float16) for _ in range(3)]
    vs = [rng.standard_normal((N, 2, 8, 4)).astype(np.float16) for _ in range(3)]
    pairs = [(1, 5), (1, 7), (2, 0)]
    k2, v2 = oracle.copy_blocks(ks, vs, pairs)
    for layer in range(3):
        for p in range(N):
            src = {5: 1, 7: 1, 0: 2}.get(p, p)
            assert np.array_equal(k2[layer][p].view(np.uint16), ks[layer][src].view(np.uint16))
            assert np.array_equal(v2[layer][p].view(np.uint16), vs[layer][src].view(np.uint16))
    with pytest.raises(ValueError):
        oracle.copy_blocks(ks, vs, [(1, 5), (2, 5)])
    with pytest.raises(ValueError):
        oracle.copy_blocks(ks, vs, [(1, 5), (5, 6)])


def _labelled_pool(labels, page_shape, nan_at=None):
    """Pool whose page i holds the binary16 value labels[i] everywhere; if
    nan_at = (page, bits), one element of that page holds that NaN bit pattern."""
    pool = np.empty((len(labels),) + page_shape, dtype=np.float16)
    for i, x in enumerate(labels):
        pool[i] = x
    if nan_at is not None:
        u = pool.view(np.uint16)
        u[(nan_at[0],) + (0,) * len(page_shape)] = nan_at[1]
    return pool


def test_swap_blocks_hand_worked():
    """Block swap between a device pool and a host reserve ("CacheFlow：基于
    llama.cpp 的多请求 LLM 推理优化引擎", section 3, block swap; section
    抢占与恢复机制, preempted blocks go to a CPU area and come back), worked by
    hand: two layers, K pages [2][4][8] and V pages [2][1][8][4]; device pages
    hold labels 10..13 (layer 0) and 20..23 (layer 1), host slots 90..92 and
    95..97; V labels are the K labels + 0.5.  One NaN payload rides along."""
    kshape, vshape = (2, 4, 8), (2, 1, 8, 4)
    dk = [_labelled_pool([10, 11, 12, 13], kshape, nan_at=(2, 0x7E15)), _labelled_pool([20, 21, 22, 23], kshape)]
    dv = [_labelled_pool([10.5, 11.5, 12.5, 13.5], vshape), _labelled_pool([20.5, 21.5, 22.5, 23.5], vshape)]
    hk = [_labelled_pool([90, 91, 92], kshape), _labelled_pool([95, 96, 97], kshape)]
    hv = [_labelled_pool([90.5, 91.5, 92.5], vshape), _labelled_pool([95.5, 96.5, 97.5], vshape)]
    dev_bits = [x.view(np.uint16).copy() for x in dk + dv]
    host_bits = [x.view(np.uint16).copy() for x in hk + hv]

    # device -> host: (device page 2 -> host slot 0), (device page 1 -> host slot 2);
    # with source and destination roles exchanged the host would read [90, 12, 10]
    nk, nv = oracle.swap_blocks(dk, dv, hk, hv, [(2, 0), (1, 2)])
    want_k = [[12, 91, 11], [22, 96, 21]]
    want_v = [[12.5, 91.5, 11.5], [22.5, 96.5, 21.5]]
    for layer in range(2):
        for slot in range(3):
            assert np.all(nv[layer][slot] == want_v[layer][slot])
            ku = nk[layer][slot].view(np.uint16).ravel()
            if layer == 0 and slot == 0:
                # the NaN payload of device page 2, element 0, is copied bit for bit
                assert ku[0] == 0x7E15 and np.all(nk[layer][slot].ravel()[1:] == 12)
            else:
                assert np.all(nk[layer][slot] == want_k[layer][slot])
    # the sources and the caller's destination arrays are left unchanged
    for x, b in zip(dk + dv, dev_bits):
        assert np.array_equal(x.view(np.uint16), b)
    for x, b in zip(hk + hv, host_bits):
        assert np.array_equal(x.view(np.uint16), b)

    # host -> device: (host slot 1 -> device page 3), (host slot 0 -> device page 1)
    bk, bv = oracle.swap_blocks(nk, nv, dk, dv, [(1, 3), (0, 1)])
    want_k = [[10, 12, 12, 91], [20, 22, 22, 96]]
    want_v = [[10.5, 12.5, 12.5, 91.5], [20.5, 22.5, 22.5, 96.5]]
    for layer in range(2):
        for page in range(4):
            assert np.all(bv[layer][page] == want_v[layer][page])
            if layer == 0 and page in (1, 2):
                # page 1 now holds what page 2 held, NaN payload included
                assert np.array_equal(bk[layer][page].view(np.uint16), dk[0][2].view(np.uint16))
            else:
                assert np.all(bk[layer][page] == want_k[layer][page])
    # a destination may appear only once
    with pytest.raises(ValueError):
        oracle.swap_blocks(dk, dv, hk, hv, [(0, 1), (2, 1)])


# ---------------------------------------------------------------- allocator

def test_allocator_golden_script():
    script = json.load(open(os.path.join(GOLD, "pool_script.json")))
    run_pool_script(oracle.AllocatorModel, script,
                    {"state": oracle.StateError, "no_pages": oracle.NoPagesError,
                     "invalid": oracle.InvalidError})


def _check_invariants(pool: oracle.AllocatorModel):
    n_free, ref = pool.stats()
    used = set()
    count = {}
    for s, pages in pool.pages.items():
        assert len(pages) == -(-pool.length[s] // pool.page_size)
        for p in pages:
            used.add(p)
            count[p] = count.get(p, 0) + 1
    assert n_free + len(used) == pool.num_pages
    assert set(pool.free).isdisjoint(used)
    for p in range(pool.num_pages):
        assert ref[p] == count.get(p, 0)


def test_allocator_random_invariants():
    rng = np.random.default_rng(10)
    pool = oracle.AllocatorModel(40, 4, rng.permutation(40))
    live = []
    for _ in range(400):
        op = rng.integers(0, 5)
        try:
            if op == 0 or not live:
                live.append(pool.seq_new())
            elif op == 1:
                pool.seq_append(live[rng.integers(len(live))], int(rng.integers(0, 9)))
            elif op == 2:
                live.append(pool.seq_fork(live[rng.integers(len(live))]))
            elif op == 3:
                s = live[rng.integers(len(live))]
                if pool.pages[s]:
                    pool.seq_cow(s, int(rng.integers(len(pool.pages[s]))))
            else:
                s = live.pop(rng.integers(len(live)))
                pool.seq_free(s)
        except (oracle.NoPagesError, oracle.StateError):
            pass
        _check_invariants(pool)
    for s in live:
        pool.seq_free(s)
    assert pool.stats()[0] == 40 and not np.any(pool.stats()[1])


def test_sharing_page_count():
    """16 sequences sharing a 64-page prefix with 8 private pages each use
    64 + 16*8 = 192 pages; without sharing 16*72 = 1152."""
    pool = oracle.AllocatorModel(2048, 128)
    s0 = pool.seq_new()
    pool.seq_append(s0, 8192)
    seqs = [s0] + [pool.seq_fork(s0) for _ in range(15)]
    for s in seqs:
        _, cow = pool.seq_append(s, 1024)
        assert cow is None          # 8192 is page aligned: no partial shared page
    assert 2048 - pool.stats()[0] == 192
    # copy-on-write of the last shared page for four sequences: four more pages
    pairs = [pool.seq_cow(s, 63) for s in seqs[:4]]
    assert len({p[0] for p in pairs}) == 1 and 2048 - pool.stats()[0] == 196
    flat = oracle.AllocatorModel(2048, 128)
    for _ in range(16):
        flat.seq_append(flat.seq_new(), 9216)
    assert 2048 - flat.stats()[0] == 1152


def test_append_cow_of_partial_shared_page():
    """P=16, a 37-token prefix shared by a fork: the first append to either side
    copies the partial page, the second side then writes in place."""
    pool = oracle.AllocatorModel(16, 16)
    a = pool.seq_new()
    pool.seq_append(a, 37)
    b = pool.seq_fork(a)
    slots, cow = pool.seq_append(b, 3)
    assert cow is not None and cow[0] == pool.pages[a][2] and cow[1] == pool.pages[b][2]
    assert list(slots) == [cow[1] * 16 + 5, cow[1] * 16 + 6, cow[1] * 16 + 7]
    slots2, cow2 = pool.seq_append(a, 1)
    assert cow2 is None and list(slots2) == [pool.pages[a][2] * 16 + 5]


# ---------------------------------------------------------------- unified span

def _row_lens(c):
    """Cells each table row holds in a prefill case (its tokens' largest kv_len)."""
    lens = np.zeros(c.block_tables.shape[0], dtype=np.int64)
    for r, kl in zip(c.token_row, c.token_kv_len):
        if r >= 0:
            lens[r] = max(lens[r], kl)
    return lens


def brute_force_unified(q, k_pool, v_pool, span, cell_seq, cell_pos, token_seq, token_pos, scale):
    """Scalar masked scan of the flat span with math.fsum / math.exp."""
    _, n_kv, P, D = k_pool.shape
    T, n_q, _ = q.shape
    G = n_q // n_kv
    sc = float(np.float32(scale))
    out = np.zeros((T, n_q, D))
    for i in range(T):
        if token_seq[i] < 0:
            continue
        cells = [c for c in range(span) if cell_seq[c] == token_seq[i] and cell_pos[c] <= token_pos[i]]
        for h in range(n_q):
            g = h // G
            z = [sc * math.fsum(float(q[i, h, d]) * float(k_pool[c // P, g, c % P, d]) for d in range(D))
                 for c in cells]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            den = math.fsum(w)
            for d in range(D):
                out[i, h, d] = math.fsum(wt * float(vcol(v_pool, c // P, g, c % P)[d])
                                         for wt, c in zip(w, cells)) / den
    return out


def test_unified_equals_paged_decode():
    """Masked scan of the span (free NaN pages included) equals the table gather."""
    c = W.tiny_decode()
    span, cs, cp = W.unified_view(c.block_tables, c.kv_lens, c.num_pages, c.page_size)
    assert span > int(c.kv_lens.sum())          # the span holds free cells as well
    S = len(c.kv_lens)
    got = oracle.unified_attention(c.q, c.k_pool, c.v_pool, span, cs, cp, np.arange(S), c.kv_lens - 1,
                                   c.scale)
    ref = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("order", ["round_robin", "grouped"])
def test_unified_equals_paged_prefill(order):
    c, k, v = _small_prefill(order=order)
    span, cs, cp = W.unified_view(c.block_tables, _row_lens(c), c.num_pages, c.page_size)
    got = oracle.unified_attention(c.q, k, v, span, cs, cp, c.token_row, c.token_pos, c.scale)
    ref = oracle.paged_attention(c.q, k, v, c.block_tables, c.token_row, c.token_kv_len,
                                 c.token_pos, c.scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_unified_brute_force_with_padding_and_free_cells():
    rng = np.random.default_rng(31)
    N, Hkv, P, D, Hq = 6, 2, 4, 8, 4
    k = rng.standard_normal((N, Hkv, P, D)).astype(np.float16)
    v_cols = rng.standard_normal((N, Hkv, D, P)).astype(np.float16)   # value columns per slot
    span = 22
    cs = rng.integers(-1, 3, size=span).astype(np.int32)   # three sequences and free cells
    cp = np.zeros(span, dtype=np.int32)
    for s in range(3):
        idx = np.nonzero(cs == s)[0]
        cp[idx] = rng.permutation(len(idx))                # positions scattered over the span
    for c in np.nonzero(cs < 0)[0]:
        k[c // P, :, c % P, :] = np.nan
        v_cols[c // P, :, :, c % P] = np.nan
    v = W.v_blocks_from_columns(v_cols)
    T = 7
    ts = np.array([0, 1, 2, -1, 0, 2, 1], dtype=np.int32)
    tp = np.array([int((cs == s).sum()) - 1 if s >= 0 else 0 for s in ts], dtype=np.int32)
    tp[4] = 1
    q = rng.standard_normal((T, Hq, D)).astype(np.float32)
    sc = np.float32(1 / math.sqrt(D))
    got = oracle.unified_attention(q, k, v, span, cs, cp, ts, tp, sc)
    ref = brute_force_unified(q, k, v, span, cs, cp, ts, tp, sc)
    assert np.all(np.isfinite(got)) and np.all(got[3] == 0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_unified_page_order_and_poison_invariance():
    """Moving the pages (with their cell labels) or replacing the poison in free
    cells by finite garbage leaves the result unchanged."""
    c = W.tiny_decode()
    S = len(c.kv_lens)
    span, cs, cp = W.unified_view(c.block_tables, c.kv_lens, c.num_pages, c.page_size)
    out = oracle.unified_attention(c.q, c.k_pool, c.v_pool, span, cs, cp, np.arange(S), c.kv_lens - 1,
                                   c.scale)
    pi = np.random.default_rng(8).permutation(c.num_pages)
    k2 = np.empty_like(c.k_pool)
    v2 = np.empty_like(c.v_pool)
    k2[pi] = c.k_pool
    v2[pi] = c.v_pool
    bt2 = np.where(c.block_tables >= 0, pi[np.maximum(c.block_tables, 0)], -1)
    span2, cs2, cp2 = W.unified_view(bt2, c.kv_lens, c.num_pages, c.page_size)
    out2 = oracle.unified_attention(c.q, k2, v2, span2, cs2, cp2, np.arange(S), c.kv_lens - 1, c.scale)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-14)
    k3 = c.k_pool.copy()
    v3 = c.v_pool.copy()
    rng = np.random.default_rng(9)
    k3[np.isnan(k3)] = rng.standard_normal(int(np.isnan(k3).sum())).astype(np.float16)
    v3[np.isnan(v3)] = rng.standard_normal(int(np.isnan(v3).sum())).astype(np.float16)
    out3 = oracle.unified_attention(c.q, k3, v3, span, cs, cp, np.arange(S), c.kv_lens - 1, c.scale)
    np.testing.assert_array_equal(out3, out)


# ---------------------------------------------------------------- swap / compaction

class _Content:
    """Simulated page contents: device page -> label, host slot -> label, moved by
    the model's copy lists exactly as the device kernels move bytes."""

    def __init__(self, m):
        self.dev = {}
        self.host = {}
        self.m = m

    def write(self, seq):
        for j, p in enumerate(self.m.pages[seq]):
            self.dev[p] = (seq, j)

    def logical(self, seq):
        return [self.dev.get(p) for p in self.m.pages[seq]]

    def to_host(self, pairs):
        for p, h in pairs:
            self.host[h] = self.dev[p]

    def to_dev(self, pairs):
        for h, p in pairs:
            self.dev[p] = self.host[h]

    def copy(self, pairs):
        snap = dict(self.dev)
        for s, d in pairs:
            self.dev[d] = snap[s]


def test_swap_out_in_round_trip_and_conservation():
    m = oracle.AllocatorModel(24, 4, np.random.default_rng(3).permutation(24))
    m.host_reserve(10)
    C = _Content(m)
    a, b = m.seq_new(), m.seq_new()
    m.seq_append(a, 17)
    m.seq_append(b, 9)
    C.write(a)
    C.write(b)
    before = C.logical(a)
    pairs = m.seq_swap_out(a)
    assert [h for _, h in pairs] == m.host[a] == [0, 1, 2, 3, 4]
    C.to_host(pairs)
    assert m.stats_host() == 10 - 5 and len(m.free) == 24 - 3
    with pytest.raises(oracle.StateError):
        m.seq_append(a, 1)
    with pytest.raises(oracle.StateError):
        m.seq_fork(a)
    with pytest.raises(oracle.StateError):
        m.block_tables([a], 8)
    c = m.seq_new()                      # reuses the freed device pages
    assert c not in (a, b)
    m.seq_append(c, 20)
    C.write(c)
    back = m.seq_swap_in(a)
    C.to_dev(back)
    assert C.logical(a) == before
    assert m.stats_host() == 10
    used = set(p for s in m.pages for p in m.pages[s])
    assert len(used) + len(m.free) == 24 and not (used & set(m.free))


def test_swap_failures_are_atomic():
    m = oracle.AllocatorModel(8, 4)
    m.host_reserve(2)
    a = m.seq_new()
    m.seq_append(a, 12)                  # 3 pages, only 2 host slots
    snap = (list(m.free), list(m.ref), {k: list(v) for k, v in m.pages.items()}, list(m.host_free))
    with pytest.raises(oracle.NoPagesError):
        m.seq_swap_out(a)
    assert (m.free, m.ref, m.pages, m.host_free) == snap
    m.host_reserve(3)
    m.seq_swap_out(a)
    b = m.seq_new()
    m.seq_append(b, 24)                  # takes 6 of the 8 pages
    snap = (list(m.free), list(m.ref), {k: list(v) for k, v in m.pages.items()}, list(m.host_free))
    with pytest.raises(oracle.NoPagesError):
        m.seq_swap_in(a)                 # needs 3, 2 free
    assert (m.free, m.ref, m.pages, m.host_free) == snap
    m.seq_free(a)                        # a swapped-out sequence can be freed
    assert m.stats_host() == 3


def test_swap_out_of_shared_pages_keeps_sharers():
    m = oracle.AllocatorModel(12, 4)
    m.host_reserve(4)
    a = m.seq_new()
    m.seq_append(a, 8)
    f = m.seq_fork(a)
    C = _Content(m)
    C.write(a)
    pairs = m.seq_swap_out(a)
    C.to_host(pairs)
    assert all(m.ref[p] == 1 for p in m.pages[f]) and len(m.free) == 10
    m.seq_append(f, 1)                   # the sharer still owns its pages
    C.to_dev(m.seq_swap_in(a))
    assert C.logical(a) == [(a, 0), (a, 1)]
    assert not (set(m.pages[a]) & set(m.pages[f]))


def test_compaction_moves_live_pages_down_and_preserves_content():
    rng = np.random.default_rng(12)
    m = oracle.AllocatorModel(32, 4, rng.permutation(32))
    C = _Content(m)
    seqs = [m.seq_new() for _ in range(5)]
    for s, n in zip(seqs, [9, 30, 4, 17, 13]):
        m.seq_append(s, n)
        C.write(s)
    f = m.seq_fork(seqs[1])
    m.seq_free(seqs[0])
    m.seq_free(seqs[3])
    before = {s: C.logical(s) for s in m.pages}
    refs = sorted(r for r in m.ref if r > 0)
    pairs = m.compact()
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts) and not (set(dsts) & {s for s, _ in pairs})
    C.copy(pairs)
    n_live = len(refs)
    assert all(p < n_live for s in m.pages for p in m.pages[s])
    assert sorted(r for r in m.ref if r > 0) == refs
    assert m.free == list(range(n_live, 32))[::-1]
    assert {s: C.logical(s) for s in m.pages} == before
    assert m.pages[f] == m.pages[seqs[1]]
    assert m.compact() == []             # already compact


# ---------------------------------------------------------------- prefix cache
# The prefix index's model is pinned against facts that do not come from the
# model's own trie: a brute-force longest common page prefix over every token
# list inserted so far, the token content each physical page really holds (a
# shared page must hold the query's tokens), conservation of references, and a
# hand-worked LRU order.

def _fill(m, content, seq, toks):
    """Appends toks to seq and records each touched page's token content."""
    P = m.page_size
    L = m.length[seq]
    _, pair = m.seq_append(seq, len(toks))
    if pair is not None:
        content[pair[1]] = content[pair[0]]
    prev = list(content.get("seq", {}).get(seq, []))[:L]   # ids are reused after a free
    assert len(prev) == L
    allt = prev + list(toks)
    content.setdefault("seq", {})[seq] = allt
    for j in range(L // P, -(-len(allt) // P)):
        content[m.pages[seq][j]] = tuple(allt[j * P:(j + 1) * P])


def _prefix_invariants(m):
    count = {}
    for pages in m.pages.values():
        for p in pages:
            count[p] = count.get(p, 0) + 1
    trie_pages = [v[2] for v in m.trie.values()]
    assert len(set(trie_pages)) == len(trie_pages)          # a page is cached once
    for p in trie_pages:
        count[p] = count.get(p, 0) + 1
    for p in range(m.num_pages):
        assert m.ref[p] == count.get(p, 0)
    assert sorted(m.free) == [p for p in range(m.num_pages) if count.get(p, 0) == 0]


def test_prefix_match_is_the_longest_cached_page_prefix():
    rng = np.random.default_rng(21)
    P = 4
    m = oracle.AllocatorModel(400, P, rng.permutation(400))
    content = {}
    # three documents sharing a 12-token head, two of them a further 8 tokens
    head = list(rng.integers(0, 50, 12))
    docs = [head + list(rng.integers(0, 50, 30)),
            head + list(rng.integers(0, 50, 30)),
            list(rng.integers(0, 50, 42))]
    docs[1][12:20] = docs[0][12:20]
    inserted = []
    for _ in range(30):
        d = docs[int(rng.integers(3))]
        n = int(rng.integers(0, len(d) + 1))
        s = m.seq_new()
        if n:
            _fill(m, content, s, d[:n])
        cut = int(rng.integers(0, n + 1))
        m.prefix_insert(s, d[:cut])
        inserted.append(d[:cut // P * P])
        if rng.random() < 0.5:
            m.seq_free(s)
        _prefix_invariants(m)
    for _ in range(60):
        d = docs[int(rng.integers(3))]
        q = d[:int(rng.integers(0, len(d) + 1))]
        if rng.random() < 0.3 and q:
            q = list(q)
            q[int(rng.integers(len(q)))] = 99          # a token no document holds
        best = 0
        for t in inserted:
            j = 0
            while (j + 1) * P <= min(len(t), len(q)) and t[j * P:(j + 1) * P] == q[j * P:(j + 1) * P]:
                j += 1
            best = max(best, j * P)
        s, matched = m.prefix_match(q)
        assert matched == best and m.length[s] == best
        for j, p in enumerate(m.pages[s]):
            assert content[p] == tuple(q[j * P:(j + 1) * P])
        _prefix_invariants(m)
        if rng.random() < 0.5:
            m.seq_free(s)


def test_prefix_eviction_order_is_least_recently_used():
    m = oracle.AllocatorModel(16, 2)        # pages handed out 0, 1, 2, ...
    seqs = {}
    for name, toks in [("a", [1, 2, 3, 4]), ("b", [5, 6, 7, 8]), ("c", [9, 10])]:
        s = m.seq_new()
        m.seq_append(s, len(toks))
        m.prefix_insert(s, toks)
        seqs[name] = s
    # a holds pages 0, 1; b holds 2, 3; c holds 4
    for s in seqs.values():
        m.seq_free(s)
    assert m.prefix_pages() == 5 and len(m.free) == 11
    t, _ = m.prefix_match([1, 2, 3, 4, 0, 0])    # a's path becomes the newest

    def evict_one():
        before = set(m.free)
        assert m.prefix_evict(1) == 1
        return (set(m.free) - before).pop()

    # b's leaf, then b's head (a leaf now, stamped with b), then c
    assert [evict_one() for _ in range(3)] == [3, 2, 4]
    assert m.prefix_evict(1) == 0                # a's pages are held by t
    m.seq_free(t)
    assert [evict_one() for _ in range(2)] == [1, 0]
    assert m.prefix_evict(1) == 0 and m.prefix_pages() == 0


def test_prefix_cache_never_evicts_a_page_in_use():
    m = oracle.AllocatorModel(12, 4)
    a = m.seq_new()
    m.seq_append(a, 16)
    m.prefix_insert(a, list(range(16)))
    b, n = m.prefix_match(list(range(8)) + [7, 7, 7, 7])
    assert n == 8 and m.pages[b] == m.pages[a][:2]
    m.seq_free(a)
    assert m.prefix_evict(10) == 2               # only a's last two pages
    assert m.prefix_pages() == 2
    assert m.prefix_capacity(0) == 0 and m.prefix_pages() == 2
    m.seq_free(b)
    assert m.prefix_pages() == 2                 # freeing b does not evict by itself
    assert m.prefix_capacity(1) == 1 and m.prefix_pages() == 1
    _prefix_invariants(m)
    assert m.prefix_capacity(0) == 1 and len(m.free) == 12


def test_prefix_capacity_bounds_the_cache_on_insert():
    m = oracle.AllocatorModel(20, 2)
    m.prefix_capacity(3)
    for k in range(4):
        s = m.seq_new()
        m.seq_append(s, 4)
        m.prefix_insert(s, [10 * k, 1, 2, 3])
        m.seq_free(s)
        assert m.prefix_pages() <= 3
        _prefix_invariants(m)
    # the newest path survives whole; older leaves went first
    _, n = m.prefix_match([30, 1, 2, 3])
    assert n == 4


def test_prefix_insert_rejects_a_page_cached_under_other_tokens():
    m = oracle.AllocatorModel(8, 2)
    a = m.seq_new()
    m.seq_append(a, 4)
    m.prefix_insert(a, [1, 2, 3, 4])
    snap = (list(m.free), list(m.ref), dict(m.trie), m.clock)
    with pytest.raises(oracle.InvalidError):
        m.prefix_insert(a, [1, 2, 9, 9])         # a's second page is cached as [3, 4]
    with pytest.raises(oracle.InvalidError):
        m.prefix_insert(a, [1, 2, 3, 4, 5])      # more tokens than a holds
    assert (m.free, m.ref, dict(m.trie), m.clock) == snap


def test_compaction_keeps_the_prefix_cache_consistent():
    rng = np.random.default_rng(22)
    P = 4
    m = oracle.AllocatorModel(40, P, rng.permutation(40))
    content = {}
    doc = list(rng.integers(0, 30, 40))
    for n in [40, 13, 27, 6]:
        s = m.seq_new()
        _fill(m, content, s, doc[:n] if n != 13 else list(rng.integers(0, 30, 13)))
        m.prefix_insert(s, content["seq"][s])
        if n != 27:
            m.seq_free(s)
    pairs = m.compact()
    snap = {}
    for sp, dp in pairs:
        snap[dp] = content[sp]
    content.update(snap)
    n_live = sum(1 for r in m.ref if r > 0)
    assert all(v[2] < n_live for v in m.trie.values())
    _prefix_invariants(m)
    s, matched = m.prefix_match(doc)
    assert matched == 40
    for j, p in enumerate(m.pages[s]):
        assert content[p] == tuple(doc[j * P:(j + 1) * P])
