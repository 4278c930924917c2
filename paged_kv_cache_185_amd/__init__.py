"""Paged attention over a block-table KV cache for AMD MI355X (gfx950).

Thin Python binding of libpa.so; every entry point has the name of its C
function in include/pa.h.  This layer only marshals arguments: torch tensors
supply device pointers and the current HIP stream, numpy arrays supply host
arrays.  All computation happens in the library's HIP kernels; if the library
is missing, every call raises.

Cache layout (one layer), binary16:
    K cache [num_pages][n_kv_heads][page_size][head_dim]
    V cache [num_pages][n_kv_heads][page_size // T][head_dim][T], T = min(page_size, 32)
            (v_slot_tile(page_size)): slots in blocks of T, each block slot-innermost
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import _lib
from ._lib import CacheDesc

__all__ = [
    "PaError", "InvalidError", "UnsupportedError", "NoPagesError", "StateError", "HipError",
    "WorkspaceError", "CacheDesc", "cache_desc", "pa_version", "pa_last_error", "Pool",
    "pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks", "pa_decode_workspace_bytes", "pa_decode",
    "pa_decode_noalloc", "pa_decode_noalloc_scratch_bytes",
    "pa_prefill_workspace_bytes", "pa_prefill", "pa_unified_workspace_bytes",
    "pa_unified_attention", "library_path",
]


class PaError(RuntimeError):
    status = None

    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class InvalidError(PaError):
    pass


class UnsupportedError(PaError):
    pass


class NoPagesError(PaError):
    pass


class StateError(PaError):
    pass


class HipError(PaError):
    pass


class WorkspaceError(PaError):
    pass


_ERR = {-1: InvalidError, -2: UnsupportedError, -3: NoPagesError, -4: StateError, -5: HipError,
        -6: WorkspaceError}


def library_path() -> str:
    return _lib.LIB_PATH


def _L():
    return _lib.load()


def _check(status: int):
    if status != 0:
        msg = _L().pa_last_error().decode(errors="replace")
        raise _ERR.get(status, PaError)(status, msg)


def pa_version() -> int:
    return int(_L().pa_version())


def pa_last_error() -> str:
    return _L().pa_last_error().decode(errors="replace")


# ---------------------------------------------------------------- helpers

def _host_i32(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a


def _i32p(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(_lib.c_i32_p)


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype, name, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")
    return ctypes.c_void_p(t.data_ptr())


def v_slot_tile(page_size: int) -> int:
    """Slots per block of a V page (the library's kVSlotTile, 32, or the page)."""
    return min(int(page_size), 32)


def v_cache_shape(num_pages: int, n_kv_heads: int, page_size: int, head_dim: int):
    """Shape of a V cache for a K cache [num_pages][n_kv_heads][page_size][head_dim]."""
    T = v_slot_tile(page_size)
    return (int(num_pages), int(n_kv_heads), int(page_size) // T, int(head_dim), T)


def cache_desc(k_cache, v_cache=None) -> CacheDesc:
    """Descriptor of a K cache [N][Hkv][P][D] (checked against V [N][Hkv][P/T][D][T])."""
    N, H, P, D = (int(x) for x in k_cache.shape)
    if v_cache is not None and tuple(v_cache.shape) != v_cache_shape(N, H, P, D):
        raise ValueError(f"V cache shape {tuple(v_cache.shape)} does not match K cache {N, H, P, D}: "
                         f"expected {v_cache_shape(N, H, P, D)}")
    return CacheDesc(N, P, H, D)


# ---------------------------------------------------------------- host pool

class Pool:
    """Host page pool / block tables (pa_pool_*)."""

    def __init__(self, num_pages: int, page_size: int, free_order: Optional[Sequence[int]] = None):
        fo = None if free_order is None else _host_i32(free_order)
        h = ctypes.c_void_p()
        _check(_L().pa_pool_create(int(num_pages), int(page_size), _i32p(fo), ctypes.byref(h)))
        self._h = h
        self.num_pages = int(num_pages)
        self.page_size = int(page_size)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _L().pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_new(self) -> int:
        s = ctypes.c_int32()
        _check(_L().pa_seq_new(self._h, ctypes.byref(s)))
        return s.value

    def seq_append(self, seq: int, n_new: int):
        slots = np.empty(max(int(n_new), 0), dtype=np.int32)
        pair = np.zeros(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_L().pa_seq_append(self._h, int(seq), int(n_new), _i32p(slots), _i32p(pair),
                                  ctypes.byref(ncow)))
        return slots, ((int(pair[0]), int(pair[1])) if ncow.value else None)

    def seq_fork(self, src: int) -> int:
        s = ctypes.c_int32()
        _check(_L().pa_seq_fork(self._h, int(src), ctypes.byref(s)))
        return s.value

    def seq_cow(self, seq: int, logical_page: int):
        pair = np.zeros(2, dtype=np.int32)
        _check(_L().pa_seq_cow(self._h, int(seq), int(logical_page), _i32p(pair)))
        return int(pair[0]), int(pair[1])

    def seq_free(self, seq: int) -> None:
        _check(_L().pa_seq_free(self._h, int(seq)))

    def block_tables(self, seqs: Sequence[int], max_pages: int):
        s = _host_i32(seqs)
        bt = np.empty((len(s), int(max_pages)), dtype=np.int32)
        kv = np.empty(len(s), dtype=np.int32)
        _check(_L().pa_block_tables(self._h, _i32p(s), len(s), int(max_pages), _i32p(bt), _i32p(kv)))
        return bt, kv

    def host_reserve(self, n_host_pages: int) -> None:
        _check(_L().pa_pool_host_reserve(self._h, int(n_host_pages)))

    def _pairs_call(self, fn, *args):
        cap = self.num_pages
        pairs = np.zeros((cap, 2), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(fn(self._h, *args, _i32p(pairs), cap, ctypes.byref(n)))
        return pairs[:n.value].copy()

    def seq_swap_out(self, seq: int) -> np.ndarray:
        """(device page, host slot) copies, in logical order; see pa_seq_swap_out."""
        return self._pairs_call(_L().pa_seq_swap_out, int(seq))

    def seq_swap_in(self, seq: int) -> np.ndarray:
        """(host slot, device page) copies, in logical order; see pa_seq_swap_in."""
        return self._pairs_call(_L().pa_seq_swap_in, int(seq))

    def compact(self) -> np.ndarray:
        """(src, dst) page moves for pa_copy_blocks; see pa_pool_compact."""
        return self._pairs_call(_L().pa_pool_compact)

    def host_free(self) -> int:
        n = ctypes.c_int32(0)
        _check(_L().pa_pool_host_stats(self._h, ctypes.byref(n)))
        return n.value

    def prefix_insert(self, seq: int, tokens: Sequence[int]) -> int:
        """Caches the sequence's full pages under their tokens; see pa_prefix_insert."""
        t = _host_i32(tokens)
        n = ctypes.c_int32(0)
        _check(_L().pa_prefix_insert(self._h, int(seq), _i32p(t), len(t), ctypes.byref(n)))
        return n.value

    def prefix_match(self, tokens: Sequence[int]):
        """(new sequence sharing the longest cached prefix, matched tokens)."""
        t = _host_i32(tokens)
        s, m = ctypes.c_int32(), ctypes.c_int32()
        _check(_L().pa_prefix_match(self._h, _i32p(t), len(t), ctypes.byref(s), ctypes.byref(m)))
        return s.value, m.value

    def prefix_evict(self, n_pages: int) -> int:
        n = ctypes.c_int32(0)
        _check(_L().pa_prefix_evict(self._h, int(n_pages), ctypes.byref(n)))
        return n.value

    def prefix_capacity(self, max_pages: int) -> int:
        n = ctypes.c_int32(0)
        _check(_L().pa_prefix_capacity(self._h, int(max_pages), ctypes.byref(n)))
        return n.value

    def prefix_pages(self) -> int:
        n = ctypes.c_int32(0)
        _check(_L().pa_prefix_stats(self._h, ctypes.byref(n)))
        return n.value

    def stats(self):
        n = ctypes.c_int32()
        ref = np.empty(self.num_pages, dtype=np.int32)
        _check(_L().pa_pool_stats(self._h, ctypes.byref(n), _i32p(ref)))
        return n.value, ref


# ---------------------------------------------------------------- device ops

def _validate_env() -> bool:
    """PA_VALIDATE as the library reads it: set and not "0"."""
    v = os.environ.get("PA_VALIDATE", "")
    return bool(v) and v[0] != "0"


def _host_copy(given, device_tensor):
    """The caller's host copy of a device table, or (under PA_VALIDATE) one
    taken from the device (a synchronizing copy), else None."""
    if given is not None:
        return _host_i32(given)
    if _validate_env():
        return _host_i32(device_tensor.cpu().numpy())
    return None


def _launch_stream(stream):
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _alloc_out_ws(q, out, workspace, need, stream):
    """The output (like q) and a zero-filled workspace of `need` bytes when the
    caller gave none, allocated on the launch stream: the zero fill is then
    ordered before the kernel, and the caching allocator does not hand the
    blocks to another stream's work while the kernel may still use them."""
    import torch
    if out is not None and (workspace is not None or need <= 0):
        return out, workspace
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None and need > 0:
            workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    return out, workspace


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def pa_reshape_and_cache(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None,
                         slot_mapping_host=None) -> None:
    """Write new tokens' K/V ([T][Hkv][D], float16 or float32) into their cells.

    ``slot_mapping_host`` (a host copy of ``slot_mapping``) lets the library
    check the slots before the launch; under PA_VALIDATE=1 it is taken from the
    device when not given."""
    import torch
    desc = cache_desc(k_cache, v_cache)
    _dev(k_cache, torch.float16, "k_cache", 4)
    _dev(v_cache, torch.float16, "v_cache", 5)
    _dev(slot_mapping, torch.int32, "slot_mapping", 1)
    T = int(slot_mapping.shape[0])
    if k_new.dtype not in (torch.float16, torch.float32) or v_new.dtype != k_new.dtype:
        raise TypeError("k_new/v_new must both be float16 or both float32")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (T, desc.n_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [{T}][{desc.n_kv_heads}][{desc.head_dim}]")
    sh = _host_copy(slot_mapping_host, slot_mapping)
    _need(sh is None or sh.shape == (T,), f"slot_mapping_host must hold {T} entries")
    _check(_L().pa_reshape_and_cache(
        ctypes.byref(desc), _dev(k_cache, torch.float16, "k_cache"),
        _dev(v_cache, torch.float16, "v_cache"), _dev(k_new, k_new.dtype, "k_new"),
        _dev(v_new, v_new.dtype, "v_new"), 1 if k_new.dtype == torch.float32 else 0,
        _dev(slot_mapping, torch.int32, "slot_mapping", 1), _i32p(sh), T, _stream_ptr(stream)))


def pa_copy_blocks(k_caches, v_caches, pairs, stream=None) -> None:
    """Copy pages src -> dst (pairs: host [n][2]) in every layer's K and V cache."""
    import torch
    if len(k_caches) != len(v_caches) or not k_caches:
        raise ValueError("need the same non-zero number of K and V caches")
    desc = cache_desc(k_caches[0], v_caches[0])
    for k, v in zip(k_caches, v_caches):
        if tuple(k.shape) != tuple(k_caches[0].shape) or tuple(v.shape) != tuple(v_caches[0].shape):
            raise ValueError("all layers must have the same cache shape")
        _dev(k, torch.float16, "k_cache", 4)
        _dev(v, torch.float16, "v_cache", 5)
    p = _host_i32(pairs).reshape(-1, 2)
    n_layers = len(k_caches)
    kp = (ctypes.c_void_p * n_layers)(*[k.data_ptr() for k in k_caches])
    vp = (ctypes.c_void_p * n_layers)(*[v.data_ptr() for v in v_caches])
    _check(_L().pa_copy_blocks(ctypes.byref(desc), kp, vp, n_layers, _i32p(p), p.shape[0],
                               _stream_ptr(stream)))


def pa_swap_blocks(k_caches, v_caches, k_host, v_host, pairs, to_host: bool, stream=None) -> None:
    """Copy whole pages between device caches and pinned host reserves of the same
    layout, per layer (pairs: host [n][2]; to_host: (device page, host slot),
    else (host slot, device page))."""
    import torch
    if not (len(k_caches) == len(v_caches) == len(k_host) == len(v_host)) or not k_caches:
        raise ValueError("need the same non-zero number of device and host K/V caches")
    desc = cache_desc(k_caches[0], v_caches[0])
    n_host = int(k_host[0].shape[0])
    for k, v, kh, vh in zip(k_caches, v_caches, k_host, v_host):
        _dev(k, torch.float16, "k_cache", 4)
        _dev(v, torch.float16, "v_cache", 5)
        for h, d in ((kh, k), (vh, v)):
            if not h.is_pinned() or h.dtype != torch.float16 or tuple(h.shape[1:]) != tuple(d.shape[1:]) \
                    or int(h.shape[0]) != n_host or not h.is_contiguous():
                raise ValueError("host reserves must be contiguous pinned float16 tensors of the cache's "
                                 "page layout")
    p = _host_i32(pairs).reshape(-1, 2)
    n_layers = len(k_caches)
    arr = lambda ts: (ctypes.c_void_p * n_layers)(*[t.data_ptr() for t in ts])   # noqa: E731
    _check(_L().pa_swap_blocks(ctypes.byref(desc), arr(k_caches), arr(v_caches), arr(k_host), arr(v_host),
                               n_host, n_layers, _i32p(p), p.shape[0], 1 if to_host else 0,
                               _stream_ptr(stream)))


def pa_decode_workspace_bytes(desc: CacheDesc, n_seqs: int, n_q_heads: int, max_pages: int,
                              kv_lens_host=None, partition_tokens: int = 0) -> int:
    kl = None if kv_lens_host is None else _host_i32(kv_lens_host)
    return int(_L().pa_decode_workspace_bytes(ctypes.byref(desc), int(n_seqs), int(n_q_heads),
                                              int(max_pages), _i32p(kl), int(partition_tokens)))


def pa_decode(q, k_cache, v_cache, block_tables, kv_lens, scale: float, kv_lens_host=None,
              partition_tokens: int = 0, out=None, workspace=None, stream=None,
              block_tables_host=None):
    """Paged decode attention; q fp32 [S][Hq][D] -> out fp32 [S][Hq][D].

    A caller-supplied ``workspace`` must be zero-filled before its first use;
    pa_decode leaves its counter region zero-filled again.  ``block_tables_host``
    (with ``kv_lens_host``) lets the library check the page ids before the
    launch; under PA_VALIDATE=1 both are taken from the device when not given."""
    import torch
    desc = cache_desc(k_cache, v_cache)
    _dev(q, torch.float32, "q", 3)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(kv_lens, torch.int32, "kv_lens", 1)
    S, Hq, D = (int(x) for x in q.shape)
    _need(D == desc.head_dim, "q head_dim does not match the cache")
    _need(int(block_tables.shape[0]) >= S, f"block_tables needs at least {S} rows")
    _need(int(kv_lens.shape[0]) == S, f"kv_lens must hold {S} entries")
    _need(out is None or tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    max_pages = int(block_tables.shape[1])
    kl = _host_copy(kv_lens_host, kv_lens)
    bh = _host_copy(block_tables_host, block_tables)
    _need(kl is None or kl.shape == (S,), f"kv_lens_host must hold {S} entries")
    _need(bh is None or bh.shape == tuple(block_tables.shape), "block_tables_host must have block_tables' shape")
    need = pa_decode_workspace_bytes(desc, S, Hq, max_pages, kl, partition_tokens)
    st = _launch_stream(stream)
    out, workspace = _alloc_out_ws(q, out, workspace, need, st)
    ws_ptr, ws_bytes = _ws_args(workspace)
    _check(_L().pa_decode(
        ctypes.byref(desc), _dev(k_cache, torch.float16, "k_cache", 4),
        _dev(v_cache, torch.float16, "v_cache", 5), _dev(q, torch.float32, "q", 3),
        _dev(out, torch.float32, "out", 3), _dev(block_tables, torch.int32, "block_tables", 2),
        _dev(kv_lens, torch.int32, "kv_lens", 1), _i32p(bh), _i32p(kl), S, max_pages, Hq, float(scale),
        int(partition_tokens), ws_ptr, ws_bytes, ctypes.c_void_p(st.cuda_stream)))
    return out


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, kv_lens, scale: float, kv_lens_host=None,
                      partition_tokens: int = 0, out=None, stream=None, block_tables_host=None):
    """pa_decode without a workspace: the split partials live in the library's
    fixed per-GPU scratch (pa_decode_noalloc_scratch_bytes()).  Allocates
    nothing when ``out`` is given.  Calls that overlap in time on one GPU race."""
    import torch
    desc = cache_desc(k_cache, v_cache)
    _dev(q, torch.float32, "q", 3)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(kv_lens, torch.int32, "kv_lens", 1)
    S, Hq, D = (int(x) for x in q.shape)
    _need(D == desc.head_dim, "q head_dim does not match the cache")
    _need(int(block_tables.shape[0]) >= S, f"block_tables needs at least {S} rows")
    _need(int(kv_lens.shape[0]) == S, f"kv_lens must hold {S} entries")
    _need(out is None or tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    kl = _host_copy(kv_lens_host, kv_lens)
    bh = _host_copy(block_tables_host, block_tables)
    _need(kl is None or kl.shape == (S,), f"kv_lens_host must hold {S} entries")
    _need(bh is None or bh.shape == tuple(block_tables.shape), "block_tables_host must have block_tables' shape")
    st = _launch_stream(stream)
    out, _ = _alloc_out_ws(q, out, None, 0, st)
    _check(_L().pa_decode_noalloc(
        ctypes.byref(desc), _dev(k_cache, torch.float16, "k_cache", 4),
        _dev(v_cache, torch.float16, "v_cache", 5), _dev(q, torch.float32, "q", 3),
        _dev(out, torch.float32, "out", 3), _dev(block_tables, torch.int32, "block_tables", 2),
        _dev(kv_lens, torch.int32, "kv_lens", 1), _i32p(bh), _i32p(kl), S, int(block_tables.shape[1]), Hq,
        float(scale), int(partition_tokens), ctypes.c_void_p(st.cuda_stream)))
    return out


def pa_decode_noalloc_scratch_bytes() -> int:
    return int(_L().pa_decode_noalloc_scratch_bytes())


def pa_prefill_workspace_bytes(desc: CacheDesc, n_q_heads: int, token_row_host, token_kv_len_host,
                               token_pos_host, kv_splits: int = 0) -> int:
    r = _host_i32(token_row_host)
    k = _host_i32(token_kv_len_host)
    p = _host_i32(token_pos_host)
    _need(r.shape == k.shape == p.shape and r.ndim == 1, "token arrays must be 1-D of one length")
    return int(_L().pa_prefill_workspace_bytes(ctypes.byref(desc), len(r), int(n_q_heads), _i32p(r),
                                               _i32p(k), _i32p(p), int(kv_splits)))


def pa_prefill(q, k_cache, v_cache, block_tables, token_row, token_kv_len, token_pos,
               scale: float, token_row_host=None, token_kv_len_host=None, token_pos_host=None,
               kv_splits: int = 0, out=None, workspace=None, stream=None, block_tables_host=None):
    """UA paged prefill; q fp32 [T][Hq][D] -> out fp32 [T][Hq][D].

    The host copies of the token arrays are taken from the device tensors if
    not given (a synchronizing copy; pass them to avoid it).  A caller-supplied
    ``workspace`` must be zero-filled before its first use (each call leaves
    its counter region zeroed again).  ``block_tables_host`` lets the library
    check the page ids before the launch; under PA_VALIDATE=1 it is taken from
    the device when not given."""
    import torch
    desc = cache_desc(k_cache, v_cache)
    _dev(q, torch.float32, "q", 3)
    _dev(block_tables, torch.int32, "block_tables", 2)
    T, Hq, D = (int(x) for x in q.shape)
    _need(D == desc.head_dim, "q head_dim does not match the cache")
    for name, t in (("token_row", token_row), ("token_kv_len", token_kv_len), ("token_pos", token_pos)):
        _dev(t, torch.int32, name, 1)
        _need(int(t.shape[0]) == T, f"{name} must hold {T} entries")
    _need(out is None or tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    rh = _host_i32(token_row.cpu().numpy() if token_row_host is None else token_row_host)
    kh = _host_i32(token_kv_len.cpu().numpy() if token_kv_len_host is None else token_kv_len_host)
    ph = _host_i32(token_pos.cpu().numpy() if token_pos_host is None else token_pos_host)
    for name, h in (("token_row_host", rh), ("token_kv_len_host", kh), ("token_pos_host", ph)):
        _need(h.shape == (T,), f"{name} must hold {T} entries")
    bh = _host_copy(block_tables_host, block_tables)
    _need(bh is None or bh.shape == tuple(block_tables.shape), "block_tables_host must have block_tables' shape")
    need = pa_prefill_workspace_bytes(desc, Hq, rh, kh, ph, kv_splits)
    st = _launch_stream(stream)
    out, workspace = _alloc_out_ws(q, out, workspace, need, st)
    ws_ptr, ws_bytes = _ws_args(workspace)
    n_rows, max_pages = (int(x) for x in block_tables.shape)
    _check(_L().pa_prefill(
        ctypes.byref(desc), _dev(k_cache, torch.float16, "k_cache", 4),
        _dev(v_cache, torch.float16, "v_cache", 5), _dev(q, torch.float32, "q", 3),
        _dev(out, torch.float32, "out", 3), _dev(block_tables, torch.int32, "block_tables", 2),
        _dev(token_row, torch.int32, "token_row", 1), _dev(token_kv_len, torch.int32, "token_kv_len", 1),
        _dev(token_pos, torch.int32, "token_pos", 1), _i32p(rh), _i32p(kh), _i32p(ph), _i32p(bh), T,
        n_rows, max_pages, Hq, float(scale), int(kv_splits), ws_ptr, ws_bytes, ctypes.c_void_p(st.cuda_stream)))
    return out


def pa_unified_workspace_bytes(desc: CacheDesc, n_tokens: int, n_q_heads: int, span: int,
                               kv_splits: int = 0) -> int:
    return int(_L().pa_unified_workspace_bytes(ctypes.byref(desc), int(n_tokens), int(n_q_heads),
                                               int(span), int(kv_splits)))


def pa_unified_attention(q, k_cache, v_cache, span: int, cell_seq, cell_pos, token_seq, token_pos,
                         scale: float, kv_splits: int = 0, out=None, workspace=None, stream=None):
    """Unified-span attention (the baseline the paged path replaces): every token
    scans cells 0..span-1 of the pool under the (cell_seq, cell_pos) mask.
    q fp32 [T][Hq][D] -> out fp32 [T][Hq][D].  Workspace rules as pa_prefill."""
    import torch
    desc = cache_desc(k_cache, v_cache)
    _dev(q, torch.float32, "q", 3)
    T, Hq, D = (int(x) for x in q.shape)
    _need(D == desc.head_dim, "q head_dim does not match the cache")
    for name, t, n in (("cell_seq", cell_seq, None), ("cell_pos", cell_pos, None), ("token_seq", token_seq, T),
                       ("token_pos", token_pos, T)):
        _dev(t, torch.int32, name, 1)
        if n is None:
            _need(int(t.shape[0]) >= int(span), f"{name} must hold at least span = {span} entries")
        else:
            _need(int(t.shape[0]) == n, f"{name} must hold {n} entries")
    _need(out is None or tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    need = pa_unified_workspace_bytes(desc, T, Hq, span, kv_splits)
    st = _launch_stream(stream)
    out, workspace = _alloc_out_ws(q, out, workspace, need, st)
    ws_ptr, ws_bytes = _ws_args(workspace)
    _check(_L().pa_unified_attention(
        ctypes.byref(desc), _dev(k_cache, torch.float16, "k_cache", 4),
        _dev(v_cache, torch.float16, "v_cache", 5), _dev(q, torch.float32, "q", 3),
        _dev(out, torch.float32, "out", 3), int(span), _dev(cell_seq, torch.int32, "cell_seq", 1),
        _dev(cell_pos, torch.int32, "cell_pos", 1), _dev(token_seq, torch.int32, "token_seq", 1),
        _dev(token_pos, torch.int32, "token_pos", 1), T, Hq, float(scale), int(kv_splits), ws_ptr,
        ws_bytes, ctypes.c_void_p(st.cuda_stream)))
    return out
