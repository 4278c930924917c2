"""reshape_and_cache and copy_blocks on the GPU: bit-exact against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_185_amd as pa
import workloads as W
from gpu_util import bits16, to_dev, to_host

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("P,D,H", [(16, 64, 2), (128, 128, 8), (32, 128, 1), (1024, 64, 2)])
def test_reshape_and_cache_f16_bitwise(P, D, H):
    rng = np.random.default_rng(P + D + H)
    N = 24
    k, v = W.nan_pools(N, H, P, D)
    T = 3 * P + 5
    kn = rng.standard_normal((T, H, D)).astype(np.float16)
    vn = rng.standard_normal((T, H, D)).astype(np.float16)
    slots = rng.choice(N * P, size=T, replace=False).astype(np.int32)
    slots[::7] = -1
    kd, vd = to_dev(k), to_dev(v)
    pa.pa_reshape_and_cache(kd, vd, to_dev(kn), to_dev(vn), to_dev(slots))
    k2, v2 = oracle.reshape_and_cache(k, v, kn, vn, slots)
    assert np.array_equal(bits16(to_host(kd)), bits16(k2))
    assert np.array_equal(bits16(to_host(vd)), bits16(v2))


def test_reshape_and_cache_f32_rounding_golden():
    g = json.load(open(os.path.join(GOLD, "f16_rounding.json")))
    bits = np.array([int(c[0], 16) for c in g["cases"]], dtype=np.uint32)
    want = np.array([int(c[1], 16) for c in g["cases"]], dtype=np.uint16)
    n = len(bits)
    D = 64
    # each case fills one whole K/V row (all D values equal) in its own page
    src = np.repeat(bits.view(np.float32)[:, None, None], D, axis=2).astype(np.float32)
    k, v = W.nan_pools(n, 1, 16, D)
    kd, vd = to_dev(k), to_dev(v)
    pa.pa_reshape_and_cache(kd, vd, to_dev(src), to_dev(src), to_dev(np.arange(n, dtype=np.int32) * 16))
    kh, vh = bits16(to_host(kd)), bits16(to_host(vd))
    for i in range(n):
        assert np.all(kh[i, 0, 0, :] == want[i]), (g["cases"][i], hex(kh[i, 0, 0, 0]))
        assert np.all(vh[i, 0, 0, :, 0] == want[i]), g["cases"][i]   # slot 0: block 0, column 0
    nan_in = np.array([int(x, 16) for x in g["nan"]], dtype=np.uint32).view(np.float32)
    src = np.repeat(nan_in[:, None, None], D, axis=2).astype(np.float32)
    k, v = W.nan_pools(len(nan_in), 1, 16, D)
    k.view(np.uint16)[...] = 0
    v.view(np.uint16)[...] = 0
    kd, vd = to_dev(k), to_dev(v)
    pa.pa_reshape_and_cache(kd, vd, to_dev(src), to_dev(src),
                            to_dev(np.arange(len(nan_in), dtype=np.int32) * 16))
    assert np.all(np.isnan(to_host(kd)[:, 0, 0, :])) and np.all(np.isnan(to_host(vd)[:, 0, 0, :, 0]))


def test_reshape_and_cache_f32_random_matches_numpy_rounding():
    rng = np.random.default_rng(3)
    N, H, P, D = 16, 4, 16, 128
    k, v = W.nan_pools(N, H, P, D)
    T = 100
    kn = (rng.standard_normal((T, H, D)) * np.exp(rng.uniform(-12, 12, (T, H, D)))).astype(np.float32)
    vn = (rng.standard_normal((T, H, D)) * 1e-5).astype(np.float32)   # many f16 subnormals
    slots = rng.choice(N * P, size=T, replace=False).astype(np.int32)
    kd, vd = to_dev(k), to_dev(v)
    pa.pa_reshape_and_cache(kd, vd, to_dev(kn), to_dev(vn), to_dev(slots))
    with np.errstate(over="ignore"):
        k2, v2 = oracle.reshape_and_cache(k, v, kn, vn, slots)
    assert np.array_equal(bits16(to_host(kd)), bits16(k2))
    assert np.array_equal(bits16(to_host(vd)), bits16(v2))


def test_reshape_and_cache_ua_ubatch():
    """The configs' mixed ubatch write: 512 interleaved tokens into a 2048-page pool."""
    c = W.ua_prefill()
    kd, vd = to_dev(c.k_pool), to_dev(c.v_pool)
    pa.pa_reshape_and_cache(kd, vd, to_dev(c.k_new), to_dev(c.v_new), to_dev(c.slot_mapping))
    k2, v2 = oracle.reshape_and_cache(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    assert np.array_equal(bits16(to_host(kd)), bits16(k2))
    assert np.array_equal(bits16(to_host(vd)), bits16(v2))


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("P,D", [(16, 64), (128, 128)])
def test_reshape_and_cache_slot_runs(f32, P, D):
    """Sequences' new tokens in page order (8-aligned runs of consecutive
    slots, written 16 bytes at a time) mixed with runs that start mid-group,
    skipped tokens inside a run and a ragged tail of the last workgroup."""
    rng = np.random.default_rng(90 + P + D + f32)
    H, N = 3, 48
    k, v = W.nan_pools(N, H, P, D)
    pages = rng.permutation(N)
    runs, used = [], 0
    for start, length in [(0, 3 * P), (5, 2 * P - 5), (P - 3, 3), (0, 61), (8, 29)]:
        pg = pages[used: used + (start + length + P - 1) // P]
        used += len(pg)
        cells = np.arange(start, start + length)
        runs.append(pg[cells // P] * P + cells % P)
    slots = np.concatenate(runs).astype(np.int32)
    slots[[9, 70, 71]] = -1
    T = len(slots)
    dt = np.float32 if f32 else np.float16
    kn = rng.standard_normal((T, H, D)).astype(dt)
    vn = rng.standard_normal((T, H, D)).astype(dt)
    kd, vd = to_dev(k), to_dev(v)
    pa.pa_reshape_and_cache(kd, vd, to_dev(kn), to_dev(vn), to_dev(slots))
    k2, v2 = oracle.reshape_and_cache(k, v, kn, vn, slots)
    assert np.array_equal(bits16(to_host(kd)), bits16(k2))
    assert np.array_equal(bits16(to_host(vd)), bits16(v2))


@pytest.mark.parametrize("n_layers", [1, 4])
def test_copy_blocks_bitwise(n_layers):
    rng = np.random.default_rng(n_layers)
    N, H, P, D = 40, 8, 128, 128
    ks = [rng.standard_normal((N, H, P, D)).astype(np.float16) for _ in range(n_layers)]
    vs = [W.v_blocks_from_columns(rng.standard_normal((N, H, D, P)).astype(np.float16)) for _ in range(n_layers)]
    for k in ks:
        k.view(np.uint16)[3] = W.NAN_F16_BITS      # NaN payloads must survive
    pairs = np.array([[3, 10], [5, 11], [5, 12], [39, 0]], dtype=np.int32)
    kd = [to_dev(k) for k in ks]
    vd = [to_dev(v) for v in vs]
    pa.pa_copy_blocks(kd, vd, pairs)
    k2, v2 = oracle.copy_blocks(ks, vs, pairs)
    for l in range(n_layers):
        assert np.array_equal(bits16(to_host(kd[l])), bits16(k2[l]))
        assert np.array_equal(bits16(to_host(vd[l])), bits16(v2[l]))


def test_copy_blocks_many_pairs_and_layers():
    """More pairs and layers than one launch carries."""
    rng = np.random.default_rng(5)
    N, H, P, D = 400, 1, 16, 64
    L = 40
    ks = [rng.standard_normal((N, H, P, D)).astype(np.float16) for _ in range(L)]
    vs = [W.v_blocks_from_columns(rng.standard_normal((N, H, D, P)).astype(np.float16)) for _ in range(L)]
    perm = rng.permutation(N)
    pairs = np.stack([perm[:150], perm[150:300]], axis=1).astype(np.int32)
    kd = [to_dev(k) for k in ks]
    vd = [to_dev(v) for v in vs]
    pa.pa_copy_blocks(kd, vd, pairs)
    k2, v2 = oracle.copy_blocks(ks, vs, pairs)
    for l in range(L):
        assert np.array_equal(bits16(to_host(kd[l])), bits16(k2[l]))
        assert np.array_equal(bits16(to_host(vd[l])), bits16(v2[l]))


def test_copy_blocks_rejects_overlap():
    k, v = W.nan_pools(8, 1, 16, 64)
    with pytest.raises(pa.InvalidError):
        pa.pa_copy_blocks([to_dev(k)], [to_dev(v)], [[1, 2], [2, 3]])


def test_empty_inputs_are_noops():
    """Zero sequences, zero tokens and zero pairs return without launching and
    leave every buffer as it was; a ubatch made only of padding tokens gives
    zero rows."""
    rng = np.random.default_rng(77)
    c = W.make_decode_case(rng, "empty", 8, 2, 64, 16, [40, 3], 12)
    kd, vd = to_dev(c.k_pool), to_dev(c.v_pool)
    D, Hq = c.head_dim, c.n_q_heads
    q0 = torch.zeros((0, Hq, D), dtype=torch.float32, device="cuda")
    bt0 = torch.zeros((0, c.block_tables.shape[1]), dtype=torch.int32, device="cuda")
    i0 = torch.zeros(0, dtype=torch.int32, device="cuda")
    out = pa.pa_decode(q0, kd, vd, bt0, i0, float(c.scale), kv_lens_host=np.zeros(0, np.int32))
    assert out.shape == (0, Hq, D)
    out = pa.pa_prefill(q0, kd, vd, to_dev(c.block_tables), i0, i0, i0, float(c.scale),
                        token_row_host=np.zeros(0, np.int32), token_kv_len_host=np.zeros(0, np.int32),
                        token_pos_host=np.zeros(0, np.int32))
    assert out.shape == (0, Hq, D)
    kn0 = torch.zeros((0, c.n_kv_heads, D), dtype=torch.float16, device="cuda")
    pa.pa_reshape_and_cache(kd, vd, kn0, kn0, i0)
    pa.pa_copy_blocks([kd], [vd], np.zeros((0, 2), np.int32))
    torch.cuda.synchronize()
    assert np.array_equal(bits16(to_host(kd)), bits16(c.k_pool))
    assert np.array_equal(bits16(to_host(vd)), bits16(c.v_pool))
    # every token of the ubatch is padding (row -1): all rows zero, finite
    T = 7
    q = torch.from_numpy(rng.standard_normal((T, Hq, D)).astype(np.float32)).cuda()
    row = np.full(T, -1, np.int32)
    kvl = np.full(T, 40, np.int32)
    pos = np.arange(T, dtype=np.int32)
    for splits in (0, 1, 2):
        got = to_host(pa.pa_prefill(q, kd, vd, to_dev(c.block_tables), to_dev(row), to_dev(kvl), to_dev(pos),
                                    float(c.scale), token_row_host=row, token_kv_len_host=kvl,
                                    token_pos_host=pos, kv_splits=splits))
        assert np.all(got == 0), splits
