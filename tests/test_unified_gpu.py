"""pa_unified_attention (the unified-span baseline) on the GPU against the oracle."""
import numpy as np
import pytest

import oracle
import paged_kv_cache_185_amd as pa
import workloads as W
from gpu_util import assert_attention_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_unified(q, kd, vd, span, cs, cp, ts, tp, scale, kv_splits=0, workspace=None):
    return to_host(pa.pa_unified_attention(to_dev(q), kd, vd, span, to_dev(cs), to_dev(cp), to_dev(ts),
                                           to_dev(tp), float(scale), kv_splits=kv_splits,
                                           workspace=workspace))


def row_lens(c):
    lens = np.zeros(c.block_tables.shape[0], dtype=np.int64)
    for r, kl in zip(c.token_row, c.token_kv_len):
        if r >= 0:
            lens[r] = max(lens[r], kl)
    return lens


@pytest.mark.parametrize("kv_splits", [0, 1, 3])
def test_unified_tiny_decode(kv_splits):
    """One query per sequence scanning a span with NaN free pages."""
    c = W.tiny_decode()
    span, cs, cp = W.unified_view(c.block_tables, c.kv_lens, c.num_pages, c.page_size)
    S = len(c.kv_lens)
    ts, tp = np.arange(S, dtype=np.int32), (c.kv_lens - 1).astype(np.int32)
    got = run_unified(c.q, to_dev(c.k_pool), to_dev(c.v_pool), span, cs, cp, ts, tp, c.scale, kv_splits)
    ref = oracle.unified_attention(c.q, c.k_pool, c.v_pool, span, cs, cp, ts, tp, c.scale)
    assert_attention_close(got, ref, f"unified tiny splits {kv_splits}")


CASES = [
    # Hq, Hkv, D, P, prefixes, new tokens, order
    (4, 2, 64, 16, [37, 20, 0], [9, 12, 40], "round_robin"),
    (32, 8, 128, 128, [300, 1000], [70, 33], "round_robin"),
    (32, 8, 128, 64, [0, 130], [200, 64], "grouped"),
    (16, 2, 128, 32, [700, 5], [33, 61], "round_robin"),
    (8, 2, 64, 256, [600, 40], [50, 20], "round_robin"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Hq{c[0]}Hkv{c[1]}D{c[2]}P{c[3]}{c[6][0]}")
@pytest.mark.parametrize("kv_splits", [0, 2])
def test_unified_matches_oracle_and_paged(case, kv_splits):
    Hq, Hkv, D, P, pre, new, order = case
    rng = np.random.default_rng(Hq + D + P + sum(pre) + 1)
    N = int(1.3 * sum((a + b + P - 1) // P for a, b in zip(pre, new))) + 4
    c = W.make_prefill_case(rng, "unified", Hq, Hkv, D, P, N, pre, new, order)
    k2, v2 = oracle.reshape_and_cache(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    kd, vd = to_dev(k2), to_dev(v2)
    span, cs, cp = W.unified_view(c.block_tables, row_lens(c), c.num_pages, c.page_size)
    got = run_unified(c.q, kd, vd, span, cs, cp, c.token_row, c.token_pos, c.scale, kv_splits)
    ref = oracle.unified_attention(c.q, k2, v2, span, cs, cp, c.token_row, c.token_pos, c.scale)
    assert_attention_close(got, ref, f"unified {case} splits {kv_splits}")
    paged = to_host(pa.pa_prefill(to_dev(c.q), kd, vd, to_dev(c.block_tables), to_dev(c.token_row),
                                  to_dev(c.token_kv_len), to_dev(c.token_pos), float(c.scale),
                                  token_row_host=c.token_row, token_kv_len_host=c.token_kv_len,
                                  token_pos_host=c.token_pos))
    assert_attention_close(got, paged.astype(np.float64), "unified vs paged")


def test_unified_padding_and_blind_tokens_get_zero_rows():
    """Padding tokens (sequence -1) and a token whose sequence has no cell in the
    span get zero rows; the others are unaffected."""
    c = W.tiny_decode()
    span, cs, cp = W.unified_view(c.block_tables, c.kv_lens, c.num_pages, c.page_size)
    ts = np.array([0, -1, 1, 7], dtype=np.int32)
    tp = np.array([c.kv_lens[0] - 1, 0, 5, 3], dtype=np.int32)
    q = np.concatenate([c.q, c.q], axis=0)[:4]
    got = run_unified(q, to_dev(c.k_pool), to_dev(c.v_pool), span, cs, cp, ts, tp, c.scale)
    ref = oracle.unified_attention(q, c.k_pool, c.v_pool, span, cs, cp, ts, tp, c.scale)
    assert np.all(got[1] == 0) and np.all(got[3] == 0)
    assert_attention_close(got, ref, "unified padding")


def test_unified_full_size_ua_ubatch_sampled():
    """The 512-token UA ubatch (8 sequences, 2K-16K prefixes) against its unified
    span (every used page of the 2048-page pool, free NaN pages in between), in
    the automatic launch configuration; oracle on every 9th token."""
    c = W.ua_prefill()
    k2, v2 = oracle.reshape_and_cache(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    span, cs, cp = W.unified_view(c.block_tables, row_lens(c), c.num_pages, c.page_size)
    assert span > int(row_lens(c).sum())
    got = run_unified(c.q, to_dev(k2), to_dev(v2), span, cs, cp, c.token_row, c.token_pos, c.scale)
    pick = np.arange(0, 512, 9)
    ref = oracle.unified_attention(c.q[pick], k2, v2, span, cs, cp, c.token_row[pick], c.token_pos[pick],
                                   c.scale)
    assert_attention_close(got[pick], ref, "unified ua")


def test_unified_deterministic_with_reused_workspace():
    import torch
    c = W.tiny_decode()
    span, cs, cp = W.unified_view(c.block_tables, c.kv_lens, c.num_pages, c.page_size)
    S = len(c.kv_lens)
    ts, tp = np.arange(S, dtype=np.int32), (c.kv_lens - 1).astype(np.int32)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    kd, vd = to_dev(c.k_pool), to_dev(c.v_pool)
    outs = [run_unified(c.q, kd, vd, span, cs, cp, ts, tp, c.scale, 3, workspace=ws) for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero()) == 0
