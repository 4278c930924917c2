#!/usr/bin/env python3
"""Benchmark: paged decode valid-KV GB/s and paged prefill TFLOP/s on one MI355X.

Decode workload (the headline value): 8 sequences x 16384 tokens, 32 query /
8 KV heads, head_dim 128, binary16 pages of 128 tokens scattered in a
2048-page pool with NaN free pages; one fp32 query per sequence.  A step is
one pa_decode call (one launch: split-KV partitions with the log-sum-exp reduce
done by the last workgroup of each sequence and KV head).
Steps rotate over `--layers` copies of the cache (distinct HBM addresses, like
the layers of a model), so no step can be served from the 256 MB last-level
cache by the previous one.  The K timed steps are one HIP graph replay (as a
serving engine replays a captured decode step).  value = valid K+V bytes x
steps / wall time between two device synchronizations; roofline.achieved =
valid bytes / (HIP-event time of the replay on the launch stream / steps).
Per-call distributions (median / p10 / p90) come from --samples back-to-back
replays of one-call graphs with an event between consecutive replays: "cold"
rotates over the cache copies, "warm" repeats one copy.
--decode-workload varlen16 / varlen128 makes the 64-sequence log-uniform batch
the headline instead (config.workload follows).

Also measured (each as per-call distributions):
* variable-length decode: 64 sequences, lengths log-uniform in [256, 32768],
  pages of 16 and of 128 tokens (one pass vs split-and-reduce per sequence);
* the UA ubatch: 512 tokens interleaved from 8 sequences after 2K-16K
  prefixes, one pa_prefill (automatic plan), against the dense f16 MFMA peak
  and against min(MFMA peak, intensity x HBM peak).

Prefill workload (reported beside it): 8 fresh sequences x 16384 tokens
prefilled in 512-token ubatches, chunk-major; each ubatch is one
pa_reshape_and_cache + one pa_prefill.  Host-side page allocation and block
tables are prepared before timing; the 256 ubatches are captured once in a HIP
graph and replayed.  Sequence s runs on stream s % --prefill-streams (default 8,
one stream per sequence; the streams fork from and join the replay stream
inside the graph): a sequence's chunks run in order, and launches of
different sequences, which share no pages, may overlap.  Each launch of this
schedule takes --prefill-splits KV splits (default 1: every (tile, KV head)
workgroup walks its whole visible range, so no launch pays split partial
stores or a combine, and the concurrent launches of other sequences fill the
compute units instead).  The last sequence's last ubatch is re-run eagerly
with the same plan after the timed replays and compared bitwise (concurrency
must not change a result).  The one-stream pass (every launch after the
previous one, with the library's automatic split plan, which fills the GPU
from one launch) is timed and reported beside it.

cpu_baseline: the float64 CPU oracle on the machine's host cores, timed on whole
decode steps of the headline batch, on four prefill ubatches spread over the
chunked pass, and on the full UA ubatch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else None
    except Exception:
        return None


def blas_info():
    """The BLAS library numpy uses and its thread count (threadpoolctl)."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"library": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "file": os.path.basename(i.get("filepath", ""))}
    except Exception:
        pass
    return None


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_hbm_traffic_8x16k.txt")
# the decode kernel and the host code that plans its launch (partition sizes, grid)
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_185_amd", "csrc", f)
                  for f in ("decode.hip", "api.cpp", "pa_internal.h")]


def decode_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


PREFILL_MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_kernel_mfma_busy_8x16k.txt")
PREFILL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_185_amd", "csrc", f)
                   for f in ("prefill.hip", "api.cpp", "pa_internal.h")]


def prefill_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in PREFILL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def prefill_mfma_busy():
    """MFMA busy fractions of the prefill kernel from the committed counter
    summary (per-launch, one dispatch at a time), or None without one or when
    the kernel or its launch planning (prefill.hip, api.cpp, pa_internal.h)
    has changed since the counters were taken."""
    import re
    try:
        with open(PREFILL_MFMA_FILE) as fh:
            text = fh.read()
        sha = re.search(r"^prefill_sources_sha256:\s*([0-9a-f]+)", text, re.M)
        if not sha or sha.group(1) != prefill_sources_sha256():
            return None
        fr = [float(x) for x in re.findall(r"MFMA busy fraction\s+([0-9.]+)", text)]
        own = re.search(r"so ([0-9.]+) of the cycles of the SIMDs it runs on", text)
        return {"automatic_split_launch_all_simds": fr[0], "unsplit_launch_all_simds": fr[1],
                "unsplit_launch_own_simds": float(own.group(1)) if own else None,
                "source": "profiles/prefill_kernel_mfma_busy_8x16k.txt"}
    except (OSError, IndexError, ValueError):
        return None


def decode_traffic():
    """Calibrated HBM bytes per decode launch (FETCH_SIZE + WRITE_SIZE) from the
    committed counter summary, or None when the decode kernel or its launch
    planning (decode.hip, api.cpp, pa_internal.h) has changed since the
    counters were taken (or there is no summary)."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("decode_sources_sha256") != decode_sources_sha256():
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def capture_graph(torch, fn, n=1):
    """fn(i, stream) for i in range(n), captured as one HIP graph on a side stream."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n):
                fn(i, torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def per_call_ms(torch, graph, calls_per_replay, n):
    """Per-call GPU time from n back-to-back replays of a graph of
    `calls_per_replay` calls, with an event recorded between consecutive
    replays on the replay stream: each sample is one replay's time divided by
    its calls (a replay of a one-call graph adds a launch gap of several
    microseconds that a serving loop's multi-call graph spreads over its
    calls).  An untimed replay goes first so the GPU is busy while the timed
    ones are enqueued."""
    stream = torch.cuda.current_stream()
    graph.replay()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        graph.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[i].elapsed_time(ev[i + 1]) / calls_per_replay for i in range(n)])


def stats_us(ms):
    us = np.asarray(ms) * 1e3
    return {"n": int(us.size), "mean_us": round(float(us.mean()), 2), "median_us": round(float(np.median(us)), 2),
            "p10_us": round(float(np.percentile(us, 10)), 2), "p90_us": round(float(np.percentile(us, 90)), 2)}


def decode_case(W, name):
    if name == "qwen3":
        return W.qwen3_decode()
    return W.varlen_decode(int(name[len("varlen"):]))   # "varlen16" / "varlen128"


def workload_text(name, c):
    if name == "qwen3":
        return ("paged decode: 8 sequences x 16384 tokens, 32 query / 8 KV heads, head_dim 128, "
                "f16 pages of 128 tokens in a 2048-page pool")
    return (f"paged decode: {len(c.kv_lens)} sequences, lengths log-uniform in [256, 32768] "
            f"(sum {int(np.sum(c.kv_lens))}), 32 query / 8 KV heads, head_dim 128, f16 pages of "
            f"{c.page_size} tokens in a {c.num_pages}-page pool")


def bench_decode(args, pa, torch, W, c):
    dev = torch.device("cuda:0")
    k0 = torch.from_numpy(c.k_pool).to(dev)
    v0 = torch.from_numpy(c.v_pool).to(dev)
    ks = [k0] + [k0.clone() for _ in range(args.layers - 1)]
    vs = [v0] + [v0.clone() for _ in range(args.layers - 1)]
    q = torch.from_numpy(c.q).to(dev)
    bt = torch.from_numpy(c.block_tables).to(dev)
    kl = torch.from_numpy(c.kv_lens).to(dev)
    out = torch.empty_like(q)
    desc = pa.cache_desc(k0, v0)
    ws_bytes = pa.pa_decode_workspace_bytes(desc, c.n_seqs, c.n_q_heads, c.block_tables.shape[1],
                                            c.kv_lens, args.partition_tokens)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def call(layer, stream):
        pa.pa_decode(q, ks[layer], vs[layer], bt, kl, float(c.scale), kv_lens_host=c.kv_lens,
                     partition_tokens=args.partition_tokens, out=out, workspace=ws, stream=stream)

    # The K timed steps are captured as one HIP graph (step i reads cache copy
    # i % layers), as a serving engine replays a whole decode step; the
    # warmup steps are a second graph replayed first.
    call(0, torch.cuda.current_stream())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if args.eager:
        run = lambda: [call(i % args.layers, stream) for i in range(args.steps)]   # noqa: E731
        for i in range(args.warmup):
            call(i % args.layers, stream)
    else:
        timed = capture_graph(torch, lambda i, st: call(i % args.layers, st), args.steps)
        if args.warmup:
            capture_graph(torch, lambda i, st: call(i % args.layers, st), args.warmup).replay()
        run = timed.replay
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms_mean = e0.elapsed_time(e1) / args.steps
    valid = W.decode_valid_bytes(c.kv_lens, c.n_kv_heads, c.head_dim)
    res = {"valid_bytes": valid, "wall_s": wall, "ms_per_step": wall * 1e3 / args.steps,
           "call_ms_mean": call_ms_mean, "workspace_bytes": ws_bytes}
    if args.samples > 0:
        k = args.calls_per_replay
        g = capture_graph(torch, lambda i, st: call(i % args.layers, st), k)
        res["cold"] = stats_us(per_call_ms(torch, g, k, args.samples))
        g = capture_graph(torch, lambda i, st: call(0, st), k)
        res["warm"] = stats_us(per_call_ms(torch, g, k, args.samples))
        del g
    return res


def gbs_block(st, nbytes):
    """A per-call distribution with the rate and HBM fraction at its median."""
    out = dict(st)
    out["GBps_at_median"] = round(nbytes / (st["median_us"] * 1e-6) / 1e9, 1)
    out["hbm_frac_at_median"] = round(nbytes / (st["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    return out


def bench_varlen(args, pa, torch, W, P):
    """64 sequences, lengths log-uniform in [256, 32768], pages of P tokens: one
    pa_decode per call on the automatic plan (partitions of at most 2048
    tokens, combined in the launch).  Every call reads ~1.76 GB, seven times
    the 256 MB last-level cache, so no rotation is needed to keep it cold."""
    c = W.varlen_decode(P)
    dev = torch.device("cuda:0")
    k = torch.from_numpy(c.k_pool).to(dev)
    v = torch.from_numpy(c.v_pool).to(dev)
    q = torch.from_numpy(c.q).to(dev)
    bt = torch.from_numpy(c.block_tables).to(dev)
    kl = torch.from_numpy(c.kv_lens).to(dev)
    out = torch.empty_like(q)
    desc = pa.cache_desc(k, v)
    ws_bytes = pa.pa_decode_workspace_bytes(desc, c.n_seqs, c.n_q_heads, c.block_tables.shape[1], c.kv_lens, 0)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def call(i, stream):
        pa.pa_decode(q, k, v, bt, kl, float(c.scale), kv_lens_host=c.kv_lens, out=out, workspace=ws,
                     stream=stream)

    call(0, torch.cuda.current_stream())
    g = capture_graph(torch, call, args.calls_per_replay)
    st = stats_us(per_call_ms(torch, g, args.calls_per_replay, args.samples))
    valid = W.decode_valid_bytes(c.kv_lens, c.n_kv_heads, c.head_dim)
    res = gbs_block(st, valid)
    res.update(valid_bytes=valid, n_seqs=int(c.n_seqs), kv_len_min=int(c.kv_lens.min()),
               kv_len_max=int(c.kv_lens.max()), kv_len_sum=int(c.kv_lens.sum()), page_size=P,
               num_pages=int(c.num_pages))
    del g, k, v
    return res


def bench_ua_ubatch(args, pa, torch, W, oracle_timer=None):
    """The UA ubatch: 512 tokens interleaved from 8 sequences (64 new tokens
    each) after prefixes of 2K-16K tokens, K/V of the new tokens written first;
    one pa_prefill per call on the automatic plan.  Cold: rotating over
    --layers copies of the pool; warm: one copy."""
    c = W.ua_prefill()
    dev = torch.device("cuda:0")
    k0, v0 = torch.from_numpy(c.k_pool).to(dev), torch.from_numpy(c.v_pool).to(dev)
    pa.pa_reshape_and_cache(k0, v0, torch.from_numpy(c.k_new).to(dev), torch.from_numpy(c.v_new).to(dev),
                            torch.from_numpy(c.slot_mapping).to(dev), slot_mapping_host=c.slot_mapping)
    ks = [k0] + [k0.clone() for _ in range(args.layers - 1)]
    vs = [v0] + [v0.clone() for _ in range(args.layers - 1)]
    q = torch.from_numpy(c.q).to(dev)
    o = torch.empty_like(q)
    bt, row = torch.from_numpy(c.block_tables).to(dev), torch.from_numpy(c.token_row).to(dev)
    kvl, pos = torch.from_numpy(c.token_kv_len).to(dev), torch.from_numpy(c.token_pos).to(dev)
    desc = pa.cache_desc(k0, v0)
    ws = torch.zeros(max(1, pa.pa_prefill_workspace_bytes(desc, c.n_q_heads, c.token_row, c.token_kv_len,
                                                          c.token_pos)), dtype=torch.uint8, device=dev)

    def call(layer, stream):
        pa.pa_prefill(q, ks[layer], vs[layer], bt, row, kvl, pos, float(c.scale), token_row_host=c.token_row,
                      token_kv_len_host=c.token_kv_len, token_pos_host=c.token_pos, out=o, workspace=ws,
                      stream=stream)

    call(0, torch.cuda.current_stream())
    k = args.calls_per_replay
    g = capture_graph(torch, lambda i, st: call(i % args.layers, st), k)
    cold = stats_us(per_call_ms(torch, g, k, args.samples))
    g = capture_graph(torch, lambda i, st: call(0, st), k)
    warm = stats_us(per_call_ms(torch, g, k, args.samples))
    del g
    pairs = W.prefill_pairs(c.token_kv_len, c.token_pos)
    flops = W.attention_flops(pairs, c.n_q_heads, c.head_dim)
    lens = np.zeros(c.block_tables.shape[0], dtype=np.int64)
    for r, n in zip(c.token_row, c.token_kv_len):
        lens[r] = max(lens[r], n)
    kv_bytes = W.decode_valid_bytes(lens, c.n_kv_heads, c.head_dim)
    intensity = flops / kv_bytes
    roof_tflops = min(MFMA_F16_PEAK_TFLOPS, intensity * HBM_PEAK_GBS / 1e3)

    def rates(st):
        tf = flops / (st["median_us"] * 1e-6) / 1e12
        return dict(st, tflops_at_median=round(tf, 1), frac_of_mfma_peak=round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                    frac_of_roofline=round(tf / roof_tflops, 4))
    return {"workload": "512 tokens interleaved round-robin from 8 sequences (64 new each) after prefixes "
                        f"{int(lens.min()) - 64}..{int(lens.max()) - 64} tokens; one pa_prefill, automatic plan",
            "flops": flops, "valid_kv_bytes": int(kv_bytes), "intensity_flop_per_byte": round(intensity, 1),
            "roofline_tflops": round(roof_tflops, 1),
            "roofline_bound": "hbm" if roof_tflops < MFMA_F16_PEAK_TFLOPS else "mfma",
            "cold": rates(cold), "warm": rates(warm)}, c


def bench_prefill(args, pa, torch, W):
    cp = W.chunked_prefill(n_seqs=8, seq_len=args.prefill_len, chunk=512, num_pages=2048)
    dev = torch.device("cuda:0")
    P, Hkv, D = cp.page_size, cp.n_kv_heads, cp.head_dim
    kc, vc = W.nan_pools(cp.num_pages, Hkv, P, D)
    kd = torch.from_numpy(kc).to(dev)
    vd = torch.from_numpy(vc).to(dev)
    del kc, vc
    qd = torch.from_numpy(cp.q).to(dev)
    knd = torch.from_numpy(cp.k).to(dev)
    vnd = torch.from_numpy(cp.v).to(dev)
    # host side: page allocation, block tables and per-token metadata for every ubatch
    pool = pa.Pool(cp.num_pages, P, cp.free_order)
    seqs = [pool.seq_new() for _ in range(cp.n_seqs)]
    max_pages = cp.seq_len // P
    plans = []
    ws_need = 0
    pairs = 0
    for s, p0 in cp.ubatches():
        n = cp.chunk
        slots, cow = pool.seq_append(seqs[s], n)
        assert cow is None
        bt, _ = pool.block_tables(seqs, max_pages)
        row = np.full(n, s, dtype=np.int32)
        kvl = np.full(n, p0 + n, dtype=np.int32)
        pos = np.arange(p0, p0 + n, dtype=np.int32)
        pairs += W.prefill_pairs(kvl, pos)
        plans.append(dict(s=s, p0=p0, n=n, slots=torch.from_numpy(slots).to(dev),
                          bt=torch.from_numpy(bt).to(dev), row=torch.from_numpy(row).to(dev),
                          kvl=torch.from_numpy(kvl).to(dev), pos=torch.from_numpy(pos).to(dev),
                          row_h=row, kvl_h=kvl, pos_h=pos))
    n_str = max(1, args.prefill_streams)
    desc = pa.cache_desc(kd, vd)
    for pl in plans:
        for sp in (0, args.prefill_splits):
            ws_need = max(ws_need, pa.pa_prefill_workspace_bytes(desc, cp.n_q_heads, pl["row_h"], pl["kvl_h"],
                                                                  pl["pos_h"], sp))
    # one workspace (split partials and counters) and one output per stream:
    # launches on different streams may run at the same time
    wss = [torch.zeros(max(ws_need, 1), dtype=torch.uint8, device=dev) for _ in range(n_str)]
    outs = [torch.empty(cp.chunk, cp.n_q_heads, D, dtype=torch.float32, device=dev) for _ in range(n_str)]
    flops = W.attention_flops(pairs, cp.n_q_heads, D)

    def prefill(pl, splits, out, ws, stream):
        s, p0, n = pl["s"], pl["p0"], pl["n"]
        pa.pa_prefill(qd[s, p0:p0 + n], kd, vd, pl["bt"], pl["row"], pl["kvl"], pl["pos"],
                      float(cp.scale), token_row_host=pl["row_h"], token_kv_len_host=pl["kvl_h"],
                      token_pos_host=pl["pos_h"], kv_splits=splits, out=out, workspace=ws, stream=stream)

    def pass_stats(per_ms):
        return {"n": int(per_ms.size), "median_ms": round(float(np.median(per_ms)), 4),
                "p10_ms": round(float(np.percentile(per_ms, 10)), 4),
                "p90_ms": round(float(np.percentile(per_ms, 90)), 4),
                "tflops_at_median": round(flops / (float(np.median(per_ms)) * 1e-3) / 1e12, 1)}

    def one_pass(streams, splits):
        # sequence s runs on stream s % len(streams): a sequence's chunks stay
        # in order, different sequences' ubatches may overlap
        for pl in plans:
            s, p0, n = pl["s"], pl["p0"], pl["n"]
            j = s % len(streams)
            pa.pa_reshape_and_cache(kd, vd, knd[s, p0:p0 + n], vnd[s, p0:p0 + n], pl["slots"],
                                    stream=streams[j])
            prefill(pl, splits, outs[j], wss[j], streams[j])

    def capture(n, splits):
        """The pass over n streams, forked from and joined back into one, as one graph."""
        streams = [torch.cuda.Stream() for _ in range(n)]
        g = torch.cuda.CUDAGraph()
        s0 = streams[0]
        s0.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s0):
            with torch.cuda.graph(g, stream=s0):
                for st in streams[1:]:
                    st.wait_stream(s0)
                one_pass(streams, splits)
                for st in streams[1:]:
                    s0.wait_stream(st)
        torch.cuda.current_stream().wait_stream(s0)
        torch.cuda.synchronize()
        return g

    def time_pass(g):
        """Mean ms per pass over --prefill-reps replays (and the wall time), plus
        the per-pass distribution of those replays (events between them)."""
        g.replay()   # warm replay
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.prefill_reps + 1)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(args.prefill_reps):
            g.replay()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.prefill_reps)])
        return ev[0].elapsed_time(ev[-1]) / args.prefill_reps, wall * 1e3 / args.prefill_reps, per

    # eager pass once (warms the code paths and fills the cache)
    one_pass([torch.cuda.current_stream()], 0)
    torch.cuda.synchronize()
    # one stream, automatic split plan: every launch waits for the previous one
    g1 = capture(1, 0)
    ms1, wall1, per1 = time_pass(g1)
    last_seq = cp.n_seqs - 1
    ref_auto = outs[0].clone()   # the last ubatch of the pass: the last sequence's last chunk
    del g1
    res = {"ubatches": len(plans), "flops": flops, "pairs": pairs, "reps": args.prefill_reps,
           "streams": n_str, "splits": args.prefill_splits, "one_stream_ms": ms1,
           "one_stream_tflops": flops / (ms1 * 1e-3) / 1e12, "one_stream_pass": pass_stats(per1)}
    g = capture(n_str, args.prefill_splits)
    ms, wall, per = time_pass(g)
    res["pass"] = pass_stats(per)
    del g
    # the last ubatch again, alone and eager, with the same plan: concurrency
    # must not change it; against the automatic plan it differs only by the
    # split combine's rounding
    got = outs[last_seq % n_str].clone()
    ref = torch.empty_like(got)
    prefill(plans[-1], args.prefill_splits, ref, wss[0], torch.cuda.current_stream())
    torch.cuda.synchronize()
    res["last_ubatch_bitwise_equal_eager"] = bool(torch.equal(ref, got))
    res["last_ubatch_max_abs_diff_vs_auto_plan"] = float((got - ref_auto).abs().max())
    res.update(pass_ms=ms, wall_ms_per_pass=wall, tflops=flops / (ms * 1e-3) / 1e12)
    return cp, plans, res


def _time_graph(torch, fn, reps):
    """Mean ms of fn() over `reps` calls captured in one HIP graph (one warm eager call first)."""
    fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(reps):
                fn(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def bench_unified(args, pa, torch, W, dec_case):
    """Paged path against the unified-span baseline on the same pool (the comparison
    the pages make end to end, here per kernel): the 512-token UA ubatch (8
    sequences, 2K-16K prefixes) and the 8 x 16384 decode batch."""
    dev = torch.device("cuda:0")
    out = {}
    # UA prefill ubatch
    c = W.ua_prefill()
    kd, vd = torch.from_numpy(c.k_pool).to(dev), torch.from_numpy(c.v_pool).to(dev)
    pa.pa_reshape_and_cache(kd, vd, torch.from_numpy(c.k_new).to(dev), torch.from_numpy(c.v_new).to(dev),
                            torch.from_numpy(c.slot_mapping).to(dev))
    lens = np.zeros(c.block_tables.shape[0], dtype=np.int64)
    for r, kl in zip(c.token_row, c.token_kv_len):
        lens[r] = max(lens[r], kl)
    span, cs, cp = W.unified_view(c.block_tables, lens, c.num_pages, c.page_size)
    q = torch.from_numpy(c.q).to(dev)
    o = torch.empty_like(q)
    bt, row = torch.from_numpy(c.block_tables).to(dev), torch.from_numpy(c.token_row).to(dev)
    kvl, pos = torch.from_numpy(c.token_kv_len).to(dev), torch.from_numpy(c.token_pos).to(dev)
    css, cps = torch.from_numpy(cs).to(dev), torch.from_numpy(cp).to(dev)
    desc = pa.cache_desc(kd, vd)
    wsp = torch.zeros(max(1, pa.pa_prefill_workspace_bytes(desc, c.n_q_heads, c.token_row, c.token_kv_len,
                                                           c.token_pos)), dtype=torch.uint8, device=dev)
    wsu = torch.zeros(max(1, pa.pa_unified_workspace_bytes(desc, len(c.token_row), c.n_q_heads, span)),
                      dtype=torch.uint8, device=dev)
    t_p = _time_graph(torch, lambda st: pa.pa_prefill(
        q, kd, vd, bt, row, kvl, pos, float(c.scale), token_row_host=c.token_row,
        token_kv_len_host=c.token_kv_len, token_pos_host=c.token_pos, out=o, workspace=wsp, stream=st), 10)
    t_u = _time_graph(torch, lambda st: pa.pa_unified_attention(
        q, kd, vd, span, css, cps, row, pos, float(c.scale), out=o, workspace=wsu, stream=st), 10)
    pairs = W.prefill_pairs(c.token_kv_len, c.token_pos)
    out["ua_prefill_512"] = {
        "paged_us": round(t_p * 1e3, 2), "unified_us": round(t_u * 1e3, 2),
        "unified_over_paged": round(t_u / t_p, 3),
        "useful_pairs": pairs, "unified_pairs": W.unified_pairs(span, len(c.token_row)),
        "span_cells": int(span), "valid_cells": int(lens.sum()),
    }
    del kd, vd
    # decode batch: the 8 queries scan the whole span together
    c = dec_case
    kd, vd = torch.from_numpy(c.k_pool).to(dev), torch.from_numpy(c.v_pool).to(dev)
    span, cs, cp = W.unified_view(c.block_tables, c.kv_lens, c.num_pages, c.page_size)
    S = len(c.kv_lens)
    q = torch.from_numpy(c.q).to(dev)
    o = torch.empty_like(q)
    bt, kl = torch.from_numpy(c.block_tables).to(dev), torch.from_numpy(c.kv_lens).to(dev)
    ts = torch.arange(S, dtype=torch.int32, device=dev)
    tp = torch.from_numpy((c.kv_lens - 1).astype(np.int32)).to(dev)
    css, cps = torch.from_numpy(cs).to(dev), torch.from_numpy(cp).to(dev)
    desc = pa.cache_desc(kd, vd)
    wsd = torch.zeros(max(1, pa.pa_decode_workspace_bytes(desc, S, c.n_q_heads, c.block_tables.shape[1],
                                                          c.kv_lens)), dtype=torch.uint8, device=dev)
    wsu = torch.zeros(max(1, pa.pa_unified_workspace_bytes(desc, S, c.n_q_heads, span)),
                      dtype=torch.uint8, device=dev)
    t_p = _time_graph(torch, lambda st: pa.pa_decode(q, kd, vd, bt, kl, float(c.scale), kv_lens_host=c.kv_lens,
                                                     out=o, workspace=wsd, stream=st), 10)
    t_u = _time_graph(torch, lambda st: pa.pa_unified_attention(
        q, kd, vd, span, css, cps, ts, tp, float(c.scale), out=o, workspace=wsu, stream=st), 10)
    out["decode_" + args.decode_workload] = {
        "paged_us": round(t_p * 1e3, 2), "unified_us": round(t_u * 1e3, 2),
        "unified_over_paged": round(t_u / t_p, 3),
        "paged_bytes": W.decode_valid_bytes(c.kv_lens, c.n_kv_heads, c.head_dim),
        "unified_bytes": W.unified_decode_bytes(span, c.n_kv_heads, c.head_dim),
        "span_cells": int(span), "valid_cells": int(np.sum(c.kv_lens)),
    }
    return out


def bench_swap_compact(args, pa, torch, W):
    """Preemption swap of one 16384-token sequence (128 pages of 512 KiB K+V) to a
    pinned host reserve and back, against a plain device<->pinned copy of the same
    bytes; and compaction of a fragmented 2048-page pool (pa_pool_compact moves,
    performed by pa_copy_blocks)."""
    dev = torch.device("cuda:0")
    P, H, D, N = 128, 8, 128, 2048
    rng = np.random.default_rng(185009)
    kd = torch.empty((N, H, P, D), dtype=torch.float16, device=dev).normal_()
    vd = torch.empty(pa.v_cache_shape(N, H, P, D), dtype=torch.float16, device=dev).normal_()
    pool = pa.Pool(N, P, rng.permutation(N))
    pool.host_reserve(256)
    seqs = [pool.seq_new() for _ in range(8)]
    for s in seqs:
        pool.seq_append(s, 16384)
    kh = torch.empty((256, H, P, D), dtype=torch.float16, pin_memory=True)
    vh = torch.empty(pa.v_cache_shape(256, H, P, D), dtype=torch.float16, pin_memory=True)
    page_bytes = 2 * H * P * D * 2
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    out_pairs = pool.seq_swap_out(seqs[0])
    pa.pa_swap_blocks([kd], [vd], [kh], [vh], out_pairs, to_host=True)       # warm
    torch.cuda.synchronize()
    e0, e1, e2 = ev(), ev(), ev()
    e0.record(stream)
    pa.pa_swap_blocks([kd], [vd], [kh], [vh], out_pairs, to_host=True)
    e1.record(stream)
    in_pairs = pool.seq_swap_in(seqs[0])
    pa.pa_swap_blocks([kd], [vd], [kh], [vh], in_pairs, to_host=False)
    e2.record(stream)
    torch.cuda.synchronize()
    nbytes = len(out_pairs) * page_bytes
    t_out, t_in = e0.elapsed_time(e1) * 1e-3, e1.elapsed_time(e2) * 1e-3
    # reference: torch's copies of the same bytes between contiguous device and pinned buffers
    dbuf = torch.empty(nbytes // 2, dtype=torch.float16, device=dev)
    hbuf = torch.empty(nbytes // 2, dtype=torch.float16, pin_memory=True)
    hbuf.copy_(dbuf, non_blocking=True)
    torch.cuda.synchronize()
    r0, r1, r2 = ev(), ev(), ev()
    r0.record(stream)
    hbuf.copy_(dbuf, non_blocking=True)
    r1.record(stream)
    dbuf.copy_(hbuf, non_blocking=True)
    r2.record(stream)
    torch.cuda.synchronize()
    ref_out, ref_in = r0.elapsed_time(r1) * 1e-3, r1.elapsed_time(r2) * 1e-3
    res = {"swap": {
        "pages": len(out_pairs), "bytes": nbytes,
        "to_host_GBps": round(nbytes / t_out / 1e9, 2), "to_device_GBps": round(nbytes / t_in / 1e9, 2),
        "plain_copy_to_host_GBps": round(nbytes / ref_out / 1e9, 2),
        "plain_copy_to_device_GBps": round(nbytes / ref_in / 1e9, 2),
    }}
    # compaction: free every other sequence of a pool filled in random page order
    for s in seqs[1::2]:
        pool.seq_free(s)
    moves = pool.compact()
    pa.pa_copy_blocks([kd], [vd], moves[:1])    # warm
    torch.cuda.synchronize()
    c0, c1 = ev(), ev()
    c0.record(stream)
    pa.pa_copy_blocks([kd], [vd], moves)
    c1.record(stream)
    torch.cuda.synchronize()
    t = c0.elapsed_time(c1) * 1e-3
    moved = len(moves) * page_bytes
    res["compaction"] = {"live_pages": int((pool.stats()[1] > 0).sum()), "moves": len(moves),
                         "bytes_moved": moved, "GBps_read_plus_write": round(2 * moved / t / 1e9, 1)}
    return res


def bench_prefix(args, pa, torch, W):
    """Admission of 16 requests that share an 8192-token prefix, each with a
    private 1024-token suffix (GQA 32/8, D 128, pages of 128 tokens), in
    512-token ubatches of reshape_and_cache + pa_prefill.  With the prefix cache,
    request 0 prefills everything and is inserted, and requests 1..15 match the
    prefix and prefill only their suffix; without it every request prefills all
    of its tokens.  Pool work (match, append, insert, tables) is host time,
    measured apart; each arm's launches are one HIP graph.  Both arms end with the
    same ubatch of the last request (same queries, lengths and K/V, different
    pages), so their outputs must be bitwise equal."""
    dev = torch.device("cuda:0")
    n_req, Lp, Ls, P, chunk = 16, 8192, 1024, 128, 512
    Hq, Hkv, D, N, vocab = 32, 8, 128, 2048, 4096
    L = Lp + Ls
    rng = np.random.default_rng(185010)
    prefix = rng.integers(0, vocab, Lp)
    tokens = [np.concatenate([prefix, rng.integers(0, vocab, Ls)]) for _ in range(n_req)]
    tkv = W.token_kv(185011, vocab, L, Hkv, D)
    ek, ev_, pk, pv = (torch.from_numpy(x).to(dev) for x in (tkv.ek, tkv.ev, tkv.pk, tkv.pv))
    tok_d = torch.from_numpy(np.stack(tokens)).to(dev)
    kn = (ek[tok_d] + pk[None]).half()               # [n_req][L][Hkv][D], as TokenKV.kv
    vn = (ev_[tok_d] + pv[None]).half()
    del ek, ev_, pk, pv
    gen = torch.Generator(device=dev)
    gen.manual_seed(185012)
    qd = torch.randn((n_req, L, Hq, D), generator=gen, device=dev, dtype=torch.float32)
    kd = torch.full((N, Hkv, P, D), float("nan"), dtype=torch.float16, device=dev)
    vd = torch.full(pa.v_cache_shape(N, Hkv, P, D), float("nan"), dtype=torch.float16, device=dev)
    desc = pa.cache_desc(kd, vd)
    free_order = rng.permutation(N)
    scale = float(W.fp32_scale(D))

    def plan(use_prefix):
        pool = pa.Pool(N, P, free_order)
        launches, host_s, pairs = [], 0.0, 0
        for r in range(n_req):
            t0 = time.perf_counter()
            if use_prefix:
                s, m = pool.prefix_match(tokens[r])
            else:
                s, m = pool.seq_new(), 0
            host_s += time.perf_counter() - t0
            for p0 in range(m, L, chunk):
                n = min(chunk, L - p0)
                t0 = time.perf_counter()
                slots, cow = pool.seq_append(s, n)
                bt, _ = pool.block_tables([s], L // P)
                host_s += time.perf_counter() - t0
                assert cow is None
                row = np.zeros(n, dtype=np.int32)
                kvl = np.full(n, p0 + n, dtype=np.int32)
                pos = np.arange(p0, p0 + n, dtype=np.int32)
                pairs += W.prefill_pairs(kvl, pos)
                launches.append(dict(r=r, p0=p0, n=n, slots=torch.from_numpy(slots).to(dev),
                                     bt=torch.from_numpy(bt).to(dev), row=torch.from_numpy(row).to(dev),
                                     kvl=torch.from_numpy(kvl).to(dev), pos=torch.from_numpy(pos).to(dev),
                                     row_h=row, kvl_h=kvl, pos_h=pos,
                                     ws=pa.pa_prefill_workspace_bytes(desc, Hq, row, kvl, pos, 0)))
            if use_prefix:
                t0 = time.perf_counter()
                pool.prefix_insert(s, tokens[r])
                host_s += time.perf_counter() - t0
        return launches, N - pool.stats()[0], host_s, pairs

    res = {"requests": n_req, "shared_prefix": Lp, "private_suffix": Ls, "ubatch": chunk}
    outs = {}
    for name, use in (("with_cache", True), ("without_cache", False)):
        launches, pages, host_s, pairs = plan(use)
        ws = torch.zeros(max(max(x["ws"] for x in launches), 1), dtype=torch.uint8, device=dev)
        out = torch.empty(chunk, Hq, D, dtype=torch.float32, device=dev)

        def one_pass(stream, launches=launches, ws=ws, out=out):
            for x in launches:
                r, p0, n = x["r"], x["p0"], x["n"]
                pa.pa_reshape_and_cache(kd, vd, kn[r, p0:p0 + n], vn[r, p0:p0 + n], x["slots"],
                                        stream=stream)
                pa.pa_prefill(qd[r, p0:p0 + n], kd, vd, x["bt"], x["row"], x["kvl"], x["pos"], scale,
                              token_row_host=x["row_h"], token_kv_len_host=x["kvl_h"],
                              token_pos_host=x["pos_h"], out=out[:n], workspace=ws, stream=stream)

        ms = _time_graph(torch, one_pass, 1)
        outs[name] = out.clone()
        flops = W.attention_flops(pairs, Hq, D)
        res[name] = {"ms": round(ms, 3), "ubatches": len(launches),
                     "tokens_prefilled": int(sum(x["n"] for x in launches)),
                     "pages_in_use": int(pages), "host_ms_pool_calls": round(host_s * 1e3, 3),
                     "attention_tflop": round(flops / 1e12, 3),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        del ws
    res["speedup"] = round(res["without_cache"]["ms"] / res["with_cache"]["ms"], 2)
    res["pages_saved"] = res["without_cache"]["pages_in_use"] - res["with_cache"]["pages_in_use"]
    res["last_ubatch_bitwise_equal"] = bool(torch.equal(outs["with_cache"].view(torch.int32),
                                                        outs["without_cache"].view(torch.int32)))
    return res


def cpu_baseline_decode(c, oracle, min_seconds=8.0, max_steps=20):
    """The oracle on whole decode steps of the batch, repeated until about
    `min_seconds` of CPU work; returns (seconds, steps)."""
    total, steps = 0.0, 0
    while steps < max_steps and (steps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        oracle.paged_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.kv_lens, c.scale)
        total += time.perf_counter() - t0
        steps += 1
    return total, steps


def cpu_baseline_prefill(cp, oracle, W, ubatch_indices=(3, 11, 19, 27)):
    """The oracle on a few ubatches of sequence 0 spread over the pass (contexts
    of 2K to 14K tokens, like the pass's mix), each with the pool filled on the
    host by the oracle's own reshape_and_cache (untimed); returns (seconds,
    algorithmic flop, description)."""
    chunk = cp.chunk
    last = cp.seq_len // chunk - 1
    js = sorted({min(j, last) for j in ubatch_indices})
    total, flops = 0.0, 0
    for j in js:
        p0 = j * chunk
        n_ctx = p0 + chunk
        n_pages = n_ctx // cp.page_size
        k, v = W.nan_pools(n_pages, cp.n_kv_heads, cp.page_size, cp.head_dim)
        slots = np.arange(n_ctx, dtype=np.int32)
        k, v = oracle.reshape_and_cache(k, v, cp.k[0, :n_ctx], cp.v[0, :n_ctx], slots)
        bt = np.arange(n_pages, dtype=np.int32)[None, :]
        row = np.zeros(chunk, np.int32)
        kvl = np.full(chunk, n_ctx, np.int32)
        pos = np.arange(p0, p0 + chunk, dtype=np.int32)
        t0 = time.perf_counter()
        oracle.paged_attention(cp.q[0, p0:p0 + chunk], k, v, bt, row, kvl, pos, cp.scale)
        total += time.perf_counter() - t0
        flops += W.attention_flops(W.prefill_pairs(kvl, pos), cp.n_q_heads, cp.head_dim)
    what = (f"sequence 0, ubatches {', '.join(str(j) for j in js)} ({chunk} tokens each, contexts "
            f"{(js[0] + 1) * chunk}..{(js[-1] + 1) * chunk})")
    return total, flops, what


def cpu_baseline_ua(c, oracle):
    """The oracle on the whole UA ubatch (all 512 tokens), over pools holding
    the new tokens' K/V (the oracle's own reshape_and_cache, untimed);
    returns seconds."""
    k, v = oracle.reshape_and_cache(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    t0 = time.perf_counter()
    oracle.paged_attention(c.q, k, v, c.block_tables, c.token_row, c.token_kv_len, c.token_pos, c.scale)
    return time.perf_counter() - t0


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=4, help="cache copies rotated over decode steps")
    ap.add_argument("--samples", type=int, default=60,
                    help="replays behind each per-call distribution (median / p10 / p90); 0 skips them")
    ap.add_argument("--calls-per-replay", type=int, default=8,
                    help="calls in the graph whose replays give the per-call distributions")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--eager", action="store_true", help="time decode steps as eager calls, not graph replays")
    ap.add_argument("--decode-workload", default="qwen3", choices=["qwen3", "varlen16", "varlen128"],
                    help="qwen3 = the 8 x 16384 headline batch; varlen* = 64 log-uniform sequences")
    ap.add_argument("--prefill-len", type=int, default=16384)
    ap.add_argument("--prefill-reps", type=int, default=50)
    ap.add_argument("--prefill-streams", type=int, default=8,
                    help="streams the prefill pass's sequences are spread over (1 = every launch in order)")
    ap.add_argument("--prefill-splits", type=int, default=1,
                    help="kv_splits of the multi-stream prefill schedule (0: the library's plan, which "
                         "fills the GPU from one launch; the one-stream pass always uses it)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-varlen", action="store_true", help="skip the variable-length decode batches")
    ap.add_argument("--no-ua", action="store_true", help="skip the UA ubatch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-unified", action="store_true",
                    help="skip the paged-vs-unified-span comparison")
    ap.add_argument("--no-swap", action="store_true", help="skip the swap / compaction measurement")
    ap.add_argument("--no-prefix", action="store_true", help="skip the prefix-cache admission measurement")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (3 times): the "
                         "known-size kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: this build measures one GPU's share of the "
              "path; how it would shard across GPUs is described, not built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_185_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_bytes} bytes 3 times")
        return
    log(f"library {pa.library_path()}")
    log(f"decode: generating the {args.decode_workload} workload")
    c = decode_case(W, args.decode_workload)
    dec = bench_decode(args, pa, torch, W, c)
    gbs = dec["valid_bytes"] * args.steps / dec["wall_s"] / 1e9
    achieved = dec["valid_bytes"] / (dec["call_ms_mean"] * 1e-3) / 1e9
    log(f"decode: {dec['call_ms_mean'] * 1e3:.1f} us/call (events), {gbs:.0f} GB/s wall")
    if "cold" in dec:
        log(f"decode per call: cold {json.dumps(dec['cold'])}, warm {json.dumps(dec['warm'])}")
    torch.cuda.empty_cache()

    varlen = {}
    if not args.no_varlen and args.samples > 0:
        for P in (16, 128):
            log(f"varlen decode P={P}")
            varlen[f"P{P}"] = bench_varlen(args, pa, torch, W, P)
            log(f"varlen decode P={P}: {json.dumps(varlen[f'P{P}'])}")
            torch.cuda.empty_cache()

    ua = ua_case = None
    if not args.no_ua and args.samples > 0:
        log("UA ubatch")
        ua, ua_case = bench_ua_ubatch(args, pa, torch, W)
        log(f"UA ubatch: {json.dumps(ua)}")
        torch.cuda.empty_cache()

    pre = None
    cp = None
    if not args.no_prefill:
        log("prefill: generating 8 x 16384 chunked workload")
        cp, _, pre = bench_prefill(args, pa, torch, W)
        log(f"prefill: {pre['pass_ms']:.2f} ms/pass, {pre['tflops']:.1f} TFLOP/s over {pre['streams']} "
            f"stream(s); one stream {pre['one_stream_ms']:.2f} ms/pass, {pre['one_stream_tflops']:.1f} TFLOP/s")
        torch.cuda.empty_cache()

    uni = None
    if not args.no_unified:
        log("unified span: paged vs unified on the UA ubatch and the decode batch")
        uni = bench_unified(args, pa, torch, W, c)
        log(f"unified span: {json.dumps(uni)}")

    swp = None
    if not args.no_swap:
        log("swap / compaction")
        swp = bench_swap_compact(args, pa, torch, W)
        log(f"swap / compaction: {json.dumps(swp)}")

    pfx = None
    if not args.no_prefix:
        log("prefix cache: 16 requests sharing an 8192-token prefix, with and without the cache")
        pfx = bench_prefix(args, pa, torch, W)
        log(f"prefix cache: {json.dumps(pfx)}")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle decode steps on the full batch")
        dt, nsteps = cpu_baseline_decode(c, oracle)
        blas = blas_info()
        cpu = {"value": dec["valid_bytes"] * nsteps / dt / 1e9, "unit": "GB/s", "kind": "oracle",
               "cores": (blas or {}).get("threads") or os.cpu_count(),
               "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "blas": blas,
               "sample": f"{nsteps} decode steps over the whole headline batch "
                         f"({len(c.kv_lens)} sequences, {int(np.sum(c.kv_lens))} tokens)",
               "seconds": dt}
        if cp is not None:
            log("cpu baseline: oracle prefill ubatches")
            dtp, fl, what = cpu_baseline_prefill(cp, oracle, W)
            cpu["prefill_tflops"] = fl / dtp / 1e12
            cpu["prefill_sample"] = what
            cpu["prefill_seconds"] = dtp
        if ua_case is not None:
            log("cpu baseline: oracle on the whole UA ubatch")
            dtu = cpu_baseline_ua(ua_case, oracle)
            cpu["ua_ubatch_seconds"] = dtu
            cpu["ua_ubatch_tflops"] = ua["flops"] / dtu / 1e12
        log(f"cpu baseline: {cpu['value']:.2f} GB/s")

    result = {
        "metric": "paged decode valid-KV GB/s (%HBM peak) + prefill TFLOP/s, 8 seqs x 16K, GQA32/8",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": workload_text(args.decode_workload, c),
            "step": "one pa_decode call over the batch; the timed steps are one HIP graph replay",
            "layers_rotated": args.layers,
            "partition_tokens": args.partition_tokens,
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "kernel": "decode_partition_kernel (the single launch of pa_decode)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": decode_traffic() if args.decode_workload == "qwen3" else None,
            "bytes_per_launch": dec["valid_bytes"],
            "call_us_mean": round(dec["call_ms_mean"] * 1e3, 2),
        },
        "cpu_baseline": cpu,
    }
    if "cold" in dec:
        result["decode_per_call"] = {
            "method": f"{dec['cold']['n']} back-to-back replays of a graph of {args.calls_per_replay} calls, an "
                      "event between consecutive replays; each sample is a replay's time / its calls",
            "cold": gbs_block(dec["cold"], dec["valid_bytes"]),
            "cold_is": f"rotating over {args.layers} cache copies (no call finds its K/V in the 256 MB "
                       "last-level cache)",
            "warm": gbs_block(dec["warm"], dec["valid_bytes"]),
            "warm_is": "the same cache copy every call",
        }
    if varlen:
        result["varlen_decode"] = varlen
    if ua is not None:
        result["ua_ubatch"] = ua
    if pre is not None:
        result["prefill"] = {
            "workload": f"8 fresh sequences x {args.prefill_len} tokens in 512-token ubatches "
                        "(reshape_and_cache + pa_prefill each), HIP-graph replay",
            "schedule": f"sequence s on stream s % {pre['streams']}, chunks of a sequence in order, "
                        f"kv_splits={pre['splits']}",
            "tflops": round(pre["tflops"], 2),
            "frac_of_mfma_f16_peak": round(pre["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
            "ms_per_pass": round(pre["pass_ms"], 4),
            "pass": pre["pass"],
            "roofline": {"kernel": "prefill_kernel (pa_prefill)", "bound": "mfma",
                         "achieved": round(pre["tflops"], 1), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(pre["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                         "basis": "algorithmic flop per pass / pass time (the schedule's launches overlap)",
                         "mfma_busy": prefill_mfma_busy()},
            "one_stream": {"schedule": "every launch after the previous one, automatic split plan",
                           "tflops": round(pre["one_stream_tflops"], 2),
                           "frac_of_mfma_f16_peak": round(pre["one_stream_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                           "ms_per_pass": round(pre["one_stream_ms"], 4),
                           "pass": pre["one_stream_pass"]},
            "flops_per_pass": pre["flops"],
            "ubatches": pre["ubatches"],
            "reps": pre["reps"],
        }
        result["prefill"]["last_ubatch_bitwise_equal_eager"] = pre["last_ubatch_bitwise_equal_eager"]
        result["prefill"]["last_ubatch_max_abs_diff_vs_auto_plan"] = pre["last_ubatch_max_abs_diff_vs_auto_plan"]
    if uni is not None:
        result["unified_vs_paged"] = uni
    if swp is not None:
        result.update(swp)
    if pfx is not None:
        result["prefix_cache"] = pfx
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
