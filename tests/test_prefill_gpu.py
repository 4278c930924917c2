"""pa_prefill (UA mixed-ubatch paged prefill) on the GPU against the oracle."""
import numpy as np
import pytest

import oracle
import paged_kv_cache_185_amd as pa
import workloads as W
from gpu_util import assert_attention_close, bits16, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_prefill(c, k_dev, v_dev, kv_splits=0, token_row=None):
    row = c.token_row if token_row is None else token_row
    out = pa.pa_prefill(to_dev(c.q), k_dev, v_dev, to_dev(c.block_tables), to_dev(row),
                        to_dev(c.token_kv_len), to_dev(c.token_pos), float(c.scale),
                        token_row_host=row, token_kv_len_host=c.token_kv_len,
                        token_pos_host=c.token_pos, kv_splits=kv_splits)
    return to_host(out)


def write_new_tokens(c):
    kd, vd = to_dev(c.k_pool), to_dev(c.v_pool)
    pa.pa_reshape_and_cache(kd, vd, to_dev(c.k_new), to_dev(c.v_new), to_dev(c.slot_mapping))
    k2, v2 = oracle.reshape_and_cache(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    assert np.array_equal(bits16(to_host(kd)), bits16(k2))
    return kd, vd, k2, v2


CASES = [
    # Hq, Hkv, D, P, prefixes, new tokens, order
    (4, 2, 64, 16, [37, 20, 0], [9, 12, 40], "round_robin"),
    (32, 8, 128, 128, [300, 1000], [70, 33], "round_robin"),
    (32, 8, 128, 64, [0, 130], [200, 64], "grouped"),
    (8, 8, 128, 16, [50, 7, 333], [17, 130, 3], "round_robin"),
    (16, 1, 64, 32, [100], [20], "grouped"),
    (16, 2, 128, 128, [700, 5], [33, 61], "round_robin"),
    (32, 4, 64, 16, [64, 65], [31, 2], "grouped"),
    (16, 4, 128, 256, [300, 0], [100, 37], "round_robin"),
    (8, 2, 64, 1024, [1100, 5], [40, 70], "grouped"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Hq{c[0]}Hkv{c[1]}D{c[2]}P{c[3]}{c[6][0]}")
@pytest.mark.parametrize("kv_splits", [0, 1, 3])
def test_prefill_shapes(case, kv_splits):
    Hq, Hkv, D, P, pre, new, order = case
    rng = np.random.default_rng(Hq + D + P + sum(pre))
    N = int(1.3 * sum((a + b + P - 1) // P for a, b in zip(pre, new))) + 4
    c = W.make_prefill_case(rng, "shape", Hq, Hkv, D, P, N, pre, new, order)
    kd, vd, k2, v2 = write_new_tokens(c)
    got = run_prefill(c, kd, vd, kv_splits)
    ref = oracle.paged_attention(c.q, k2, v2, c.block_tables, c.token_row, c.token_kv_len,
                                 c.token_pos, c.scale)
    assert_attention_close(got, ref, f"{case} splits {kv_splits}")


def test_padding_tokens_get_zero_rows():
    rng = np.random.default_rng(21)
    c = W.make_prefill_case(rng, "pad", 8, 2, 64, 16, 40, [30, 50], [10, 14], "round_robin")
    kd, vd, k2, v2 = write_new_tokens(c)
    row = c.token_row.copy()
    row[[0, 5, 23]] = -1
    for splits in (1, 3):
        got = run_prefill(c, kd, vd, splits, token_row=row)
        ref = oracle.paged_attention(c.q, k2, v2, c.block_tables, row, c.token_kv_len,
                                     c.token_pos, c.scale)
        assert np.all(got[[0, 5, 23]] == 0)
        assert_attention_close(got, ref, f"padding splits {splits}")


def test_prefill_of_last_tokens_equals_decode():
    """One token per sequence at position L-1 is a decode step."""
    c = W.tiny_decode()
    kd, vd = to_dev(c.k_pool), to_dev(c.v_pool)
    dec = to_host(pa.pa_decode(to_dev(c.q), kd, vd, to_dev(c.block_tables), to_dev(c.kv_lens),
                               float(c.scale), kv_lens_host=c.kv_lens))
    rows = np.array([1, 0], dtype=np.int32)
    pre = to_host(pa.pa_prefill(to_dev(c.q[::-1].copy()), kd, vd, to_dev(c.block_tables),
                                to_dev(rows), to_dev(c.kv_lens[rows]), to_dev(c.kv_lens[rows] - 1),
                                float(c.scale), token_row_host=rows,
                                token_kv_len_host=c.kv_lens[rows],
                                token_pos_host=c.kv_lens[rows] - 1))
    # decode carries Q to ~22 bits, prefill rounds Q to binary16: compare at the
    # attention tolerance, both against the oracle and against each other
    ref = oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
    assert_attention_close(pre[::-1], ref, "prefill as decode")
    assert_attention_close(pre[::-1], dec.astype(np.float64), "prefill vs decode")


def test_prefill_deterministic_and_permutation_invariant():
    rng = np.random.default_rng(22)
    c = W.make_prefill_case(rng, "perm", 32, 8, 128, 16, 120, [200, 90], [40, 24], "round_robin")
    kd, vd, k2, v2 = write_new_tokens(c)
    a = run_prefill(c, kd, vd, 3)
    assert np.array_equal(a, run_prefill(c, kd, vd, 3))
    pi = rng.permutation(c.num_pages)
    kp = np.empty_like(k2)
    vp = np.empty_like(v2)
    kp[pi] = k2
    vp[pi] = v2
    bt = np.where(c.block_tables >= 0, pi[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    out = pa.pa_prefill(to_dev(c.q), to_dev(kp), to_dev(vp), to_dev(bt), to_dev(c.token_row),
                        to_dev(c.token_kv_len), to_dev(c.token_pos), float(c.scale),
                        token_row_host=c.token_row, token_kv_len_host=c.token_kv_len,
                        token_pos_host=c.token_pos, kv_splits=3)
    assert np.array_equal(a, to_host(out))


def test_ua_prefill_full_size():
    """512 tokens interleaved from 8 sequences after 2K-16K prefixes, every
    output element against the oracle, in the automatic launch configuration
    (the one the benchmark times) and unsplit."""
    c = W.ua_prefill()
    kd, vd, k2, v2 = write_new_tokens(c)
    ref = oracle.paged_attention(c.q, k2, v2, c.block_tables, c.token_row, c.token_kv_len,
                                 c.token_pos, c.scale)
    assert_attention_close(run_prefill(c, kd, vd, 0), ref, "UA ubatch 512 tokens, automatic splits")
    assert_attention_close(run_prefill(c, kd, vd, 1), ref, "UA ubatch 512 tokens, unsplit")


def test_chunked_prefill_sampled_ubatches():
    """Fresh sequences prefilled in 512-token ubatches (the throughput workload),
    shortened to 2 sequences x 4096 tokens; every ubatch runs, the oracle checks
    the first, a middle and the last ubatch on sampled tokens."""
    cp = W.chunked_prefill(n_seqs=2, seq_len=4096, chunk=512, num_pages=128)
    P, Hkv, D = cp.page_size, cp.n_kv_heads, cp.head_dim
    pool = pa.Pool(cp.num_pages, P, cp.free_order)
    model = oracle.AllocatorModel(cp.num_pages, P, cp.free_order)
    seqs = [pool.seq_new() for _ in range(cp.n_seqs)]
    assert seqs == [model.seq_new() for _ in range(cp.n_seqs)]
    k_pool, v_pool = W.nan_pools(cp.num_pages, Hkv, P, D)
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    max_pages = cp.seq_len // P
    checks = {0, 5, 15}
    for j, (s, p0) in enumerate(cp.ubatches()):
        n = cp.chunk
        slots, cow = pool.seq_append(seqs[s], n)
        mslots, _ = model.seq_append(seqs[s], n)
        assert cow is None and np.array_equal(slots, mslots)
        pa.pa_reshape_and_cache(kd, vd, to_dev(cp.k[s, p0:p0 + n]), to_dev(cp.v[s, p0:p0 + n]),
                                to_dev(slots))
        k_pool, v_pool = oracle.reshape_and_cache(k_pool, v_pool, cp.k[s, p0:p0 + n],
                                                  cp.v[s, p0:p0 + n], mslots)
        bt, kv = pool.block_tables(seqs, max_pages)
        mbt, _ = model.block_tables(seqs, max_pages)
        assert np.array_equal(bt, mbt)
        row = np.full(n, s, dtype=np.int32)
        kvl = np.full(n, p0 + n, dtype=np.int32)
        pos = np.arange(p0, p0 + n, dtype=np.int32)
        out = pa.pa_prefill(to_dev(cp.q[s, p0:p0 + n]), kd, vd, to_dev(bt), to_dev(row),
                            to_dev(kvl), to_dev(pos), float(cp.scale), token_row_host=row,
                            token_kv_len_host=kvl, token_pos_host=pos)
        if j in checks:
            got = to_host(out)
            pick = np.array([0, 1, 63, 64, 200, 311, 510, 511])
            ref = oracle.paged_attention(cp.q[s, p0:p0 + n][pick], k_pool, v_pool, mbt, row[pick],
                                         kvl[pick], pos[pick], cp.scale)
            assert_attention_close(got[pick], ref, f"ubatch {j}")
    assert np.array_equal(bits16(to_host(kd)), bits16(k_pool))


def test_workspace_reused_across_calls_and_shapes():
    """Split tiles count their finished splits in the workspace's counter
    region and the combining split zeroes it again, so one zero-filled
    workspace serves calls of different shapes and split counts, and a
    repeated call reproduces its first result bitwise (the splits are folded
    in a fixed order whichever finishes last)."""
    import torch
    shapes = [(32, 8, 128, 128, [3000, 1000], [70, 33], 3),
              (8, 2, 64, 16, [900, 50, 400], [40, 12, 7], 0),
              (16, 4, 128, 64, [2500], [130], 5)]
    cases = []
    for i, (Hq, Hkv, D, P, pre, new, ks) in enumerate(shapes):
        rng = np.random.default_rng(60 + i)
        N = int(1.3 * sum((a + b + P - 1) // P for a, b in zip(pre, new))) + 4
        c = W.make_prefill_case(rng, "ws", Hq, Hkv, D, P, N, pre, new, "round_robin")
        kd, vd, k2, v2 = write_new_tokens(c)
        ref = oracle.paged_attention(c.q, k2, v2, c.block_tables, c.token_row, c.token_kv_len,
                                     c.token_pos, c.scale)
        cases.append((c, kd, vd, ks, ref))
    ws = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    first = {}
    for rep in range(3):
        for i, (c, kd, vd, ks, ref) in enumerate(cases):
            need = pa.pa_prefill_workspace_bytes(pa.cache_desc(kd, vd), c.q.shape[1], c.token_row,
                                                 c.token_kv_len, c.token_pos, ks)
            assert 0 < need <= ws.numel()
            out = to_host(pa.pa_prefill(to_dev(c.q), kd, vd, to_dev(c.block_tables),
                                        to_dev(c.token_row), to_dev(c.token_kv_len),
                                        to_dev(c.token_pos), float(c.scale),
                                        token_row_host=c.token_row, token_kv_len_host=c.token_kv_len,
                                        token_pos_host=c.token_pos, kv_splits=ks, workspace=ws))
            if rep == 0:
                assert_attention_close(out, ref, f"prefill reuse {i}")
                first[i] = out
            else:
                assert np.array_equal(out, first[i]), f"prefill reuse {i} rep {rep}"
    torch.cuda.synchronize()
    assert int(ws[:65536].count_nonzero()) == 0


@pytest.mark.parametrize("kv_splits", [1, 2])
def test_chunked_prefill_concurrent_streams_bitwise(kv_splits):
    """Sequences prefilled concurrently, sequence s on stream s (its chunks in
    order on that stream, each stream with its own workspace), give bitwise
    the outputs of the same launches run one after another; sampled tokens of
    the last ubatch of each sequence are checked against the oracle."""
    import torch
    cp = W.chunked_prefill(n_seqs=4, seq_len=2048, chunk=512, num_pages=160)
    P, Hkv, D = cp.page_size, cp.n_kv_heads, cp.head_dim
    pool = pa.Pool(cp.num_pages, P, cp.free_order)
    seqs = [pool.seq_new() for _ in range(cp.n_seqs)]
    k_pool, v_pool = W.nan_pools(cp.num_pages, Hkv, P, D)
    max_pages = cp.seq_len // P
    ubs = []
    for s, p0 in cp.ubatches():
        n = cp.chunk
        slots, cow = pool.seq_append(seqs[s], n)
        assert cow is None
        bt, _ = pool.block_tables(seqs, max_pages)
        row = np.full(n, s, dtype=np.int32)
        kvl = np.full(n, p0 + n, dtype=np.int32)
        pos = np.arange(p0, p0 + n, dtype=np.int32)
        ubs.append(dict(s=s, p0=p0, slots=slots, bt=bt, row=row, kvl=kvl, pos=pos,
                        dev=[to_dev(x) for x in (slots, bt, row, kvl, pos)]))
    q = to_dev(cp.q)
    kn, vn = to_dev(cp.k), to_dev(cp.v)

    def run(streams):
        kd, vd = to_dev(k_pool), to_dev(v_pool)
        need = max(pa.pa_prefill_workspace_bytes(pa.cache_desc(kd, vd), cp.n_q_heads, u["row"], u["kvl"],
                                                 u["pos"], kv_splits) for u in ubs)
        ws = [torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda") for _ in streams]
        # the zero fill (and the pool upload) ran on the current stream
        for st in streams:
            st.wait_stream(torch.cuda.current_stream())
        outs = []
        for u in ubs:
            s, p0, n = u["s"], u["p0"], cp.chunk
            j = s % len(streams)
            slots, bt, row, kvl, pos = u["dev"]
            pa.pa_reshape_and_cache(kd, vd, kn[s, p0:p0 + n], vn[s, p0:p0 + n], slots, stream=streams[j])
            out = torch.empty(n, cp.n_q_heads, D, dtype=torch.float32, device="cuda")
            pa.pa_prefill(q[s, p0:p0 + n], kd, vd, bt, row, kvl, pos, float(cp.scale),
                          token_row_host=u["row"], token_kv_len_host=u["kvl"], token_pos_host=u["pos"],
                          kv_splits=kv_splits, out=out, workspace=ws[j], stream=streams[j])
            outs.append(out)
        torch.cuda.synchronize()
        return [to_host(o) for o in outs], to_host(kd)

    seq_outs, kseq = run([torch.cuda.current_stream()])
    conc_outs, kconc = run([torch.cuda.Stream() for _ in range(cp.n_seqs)])
    assert np.array_equal(bits16(kseq), bits16(kconc))
    for j, (a, b) in enumerate(zip(seq_outs, conc_outs)):
        assert np.array_equal(a, b), f"ubatch {j}"
    kh, vh = k_pool, v_pool
    for u in ubs:
        s, p0, n = u["s"], u["p0"], cp.chunk
        kh, vh = oracle.reshape_and_cache(kh, vh, cp.k[s, p0:p0 + n], cp.v[s, p0:p0 + n], u["slots"])
    pick = np.array([0, 17, 255, 256, 511])
    for j, u in enumerate(ubs):
        if u["p0"] + cp.chunk != cp.seq_len:
            continue
        s, p0 = u["s"], u["p0"]
        ref = oracle.paged_attention(cp.q[s, p0:p0 + cp.chunk][pick], kh, vh, u["bt"], u["row"][pick],
                                     u["kvl"][pick], u["pos"][pick], cp.scale)
        assert_attention_close(conc_outs[j][pick], ref, f"sequence {s} last ubatch")


def test_chunked_prefill_full_size_in_both_benchmark_schedules():
    """The timed prefill pass at full size (8 sequences x 16384 tokens, 512-token
    ubatches) in the two launch configurations the benchmark times: (a) sequence
    s on stream s, unsplit launches (kv_splits = 1), captured in one HIP graph
    and replayed; (b) one stream, the library's automatic split plan.  Every
    output element of the first, a middle and the last ubatch (contexts 512,
    8704 and 16384) is checked against the oracle, computed over a private host
    pool of the ubatch's sequence."""
    import torch
    cp = W.chunked_prefill()
    P, Hkv, D = cp.page_size, cp.n_kv_heads, cp.head_dim
    pool = pa.Pool(cp.num_pages, P, cp.free_order)
    seqs = [pool.seq_new() for _ in range(cp.n_seqs)]
    k_pool, v_pool = W.nan_pools(cp.num_pages, Hkv, P, D)
    kd, vd = to_dev(k_pool), to_dev(v_pool)
    del k_pool, v_pool
    qd, knd, vnd = to_dev(cp.q), to_dev(cp.k), to_dev(cp.v)
    max_pages = cp.seq_len // P
    ubs = []
    for s, p0 in cp.ubatches():
        n = cp.chunk
        slots, cow = pool.seq_append(seqs[s], n)
        assert cow is None
        bt, _ = pool.block_tables(seqs, max_pages)
        row = np.full(n, s, np.int32)
        kvl = np.full(n, p0 + n, np.int32)
        pos = np.arange(p0, p0 + n, dtype=np.int32)
        ubs.append(dict(s=s, p0=p0, row=row, kvl=kvl, pos=pos,
                        dev=[to_dev(x) for x in (slots, bt, row, kvl, pos)]))
    check = [0, len(ubs) // 2 + 3, len(ubs) - 1]
    new_out = lambda: torch.empty(cp.chunk, cp.n_q_heads, D, dtype=torch.float32, device="cuda")  # noqa: E731
    outs = {sched: {j: new_out() for j in check} for sched in ("streams", "one")}
    scratch = [new_out() for _ in range(cp.n_seqs)]

    def launch(j, stream, splits, out, ws=None):
        u = ubs[j]
        s, p0, n = u["s"], u["p0"], cp.chunk
        slots, bt, row, kvl, pos = u["dev"]
        pa.pa_reshape_and_cache(kd, vd, knd[s, p0:p0 + n], vnd[s, p0:p0 + n], slots, stream=stream)
        pa.pa_prefill(qd[s, p0:p0 + n], kd, vd, bt, row, kvl, pos, float(cp.scale),
                      token_row_host=u["row"], token_kv_len_host=u["kvl"], token_pos_host=u["pos"],
                      kv_splits=splits, out=out, workspace=ws, stream=stream)

    # (a) one stream per sequence, unsplit, one graph
    streams = [torch.cuda.Stream() for _ in range(cp.n_seqs)]
    g = torch.cuda.CUDAGraph()
    s0 = streams[0]
    s0.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s0):
        with torch.cuda.graph(g, stream=s0):
            for st in streams[1:]:
                st.wait_stream(s0)
            for j, u in enumerate(ubs):
                launch(j, streams[u["s"]], 1, outs["streams"].get(j, scratch[u["s"]]))
            for st in streams[1:]:
                s0.wait_stream(st)
    torch.cuda.current_stream().wait_stream(s0)
    g.replay()
    torch.cuda.synchronize()
    del g
    # (b) one stream, automatic split plan (rewrites the same K/V bits)
    stream = torch.cuda.current_stream()
    need = max(pa.pa_prefill_workspace_bytes(pa.cache_desc(kd, vd), cp.n_q_heads, u["row"], u["kvl"], u["pos"], 0)
               for u in ubs)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    for j in range(len(ubs)):
        launch(j, stream, 0, outs["one"].get(j, scratch[0]), ws)
    torch.cuda.synchronize()
    for j in check:
        u = ubs[j]
        s, p0, n = u["s"], u["p0"], cp.chunk
        n_ctx = p0 + n
        kh, vh = W.nan_pools(n_ctx // P, Hkv, P, D)
        kh, vh = oracle.reshape_and_cache(kh, vh, cp.k[s, :n_ctx], cp.v[s, :n_ctx],
                                          np.arange(n_ctx, dtype=np.int32))
        bt_priv = np.arange(n_ctx // P, dtype=np.int32)[None, :]
        ref = oracle.paged_attention(cp.q[s, p0:p0 + n], kh, vh, bt_priv, np.zeros(n, np.int32),
                                     u["kvl"], u["pos"], cp.scale)
        del kh, vh
        for sched, what in (("streams", "8 streams, kv_splits=1, graph"), ("one", "one stream, automatic splits")):
            assert_attention_close(to_host(outs[sched][j]), ref,
                                   f"8x16384 pass ubatch {j} (sequence {s}, context {n_ctx}), {what}")


@pytest.mark.parametrize("kv_splits", [1, 0])
def test_prefill_range_longer_than_one_split_page_table(kv_splits):
    """Tokens whose visible range (about 140000 keys at P = 16, 8750 pages) is
    more than one workgroup stages: even an unsplit request is cut at the
    staged-table limit and combined."""
    rng = np.random.default_rng(140001)
    pre, new = [140000 - 40], [40]
    N = (140000 + 15) // 16 + 64
    c = W.make_prefill_case(rng, "long", 8, 2, 64, 16, N, pre, new, "grouped")
    kd, vd, k2, v2 = write_new_tokens(c)
    got = run_prefill(c, kd, vd, kv_splits)
    pick = np.array([0, 1, 17, 38, 39])
    ref = oracle.paged_attention(c.q[pick], k2, v2, c.block_tables, c.token_row[pick],
                                 c.token_kv_len[pick], c.token_pos[pick], c.scale)
    assert_attention_close(got[pick], ref, f"long range splits {kv_splits}")
