"""ctypes binding of libzp.so (the C ABI declared in include/zp.h).

Argument marshalling only: tensors are passed as device pointers
(``Tensor.data_ptr()``), streams as their hipStream_t handle, host arrays as
NumPy int32 buffers.  Every computation happens in the library's HIP kernels.
There is deliberately no fallback: if the library is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ZP_LIBRARY names another build of the same library (the host-side
# sanitizer test loads an instrumented one); by default the in-tree build.
LIB_PATH = os.environ.get("ZP_LIBRARY") or os.path.join(HERE, "libzp.so")

ZP_OK, ZP_ERR_INVALID, ZP_ERR_NO_BLOCKS, ZP_ERR_HIP, ZP_ERR_STATE = range(5)
ZP_F32, ZP_BF16 = 0, 1
ZP_POOL_MANUAL_FENCE = 1

_STATUS_NAMES = {0: "ZP_OK", 1: "ZP_ERR_INVALID", 2: "ZP_ERR_NO_BLOCKS", 3: "ZP_ERR_HIP",
                 4: "ZP_ERR_STATE"}


class ZpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _KVCache(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_cache", ctypes.POINTER(ctypes.c_void_p)),
                ("v_cache", ctypes.POINTER(ctypes.c_void_p))]


class _SchedConfig(ctypes.Structure):
    _fields_ = [("n_max", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("window", ctypes.c_int32), ("num_query_slots", ctypes.c_int32),
                ("max_running", ctypes.c_int32), ("prefill_chunk", ctypes.c_int32)]


_i64p_t = ctypes.POINTER(ctypes.c_int64)
_i32p_t = ctypes.POINTER(ctypes.c_int32)


class _SchedStep(ctypes.Structure):
    _fields_ = [("num_admitted", ctypes.c_int32), ("admitted", _i64p_t),
                ("num_decode", ctypes.c_int32), ("decode_ids", _i64p_t),
                ("decode_slot", _i32p_t), ("decode_seq_len", _i32p_t),
                ("decode_record_row", _i32p_t),
                ("num_compress", ctypes.c_int32), ("compress_ids", _i64p_t),
                ("compress_qslot", _i32p_t), ("compress_n_src", _i32p_t),
                ("num_prefill", ctypes.c_int32), ("prefill_ids", _i64p_t),
                ("prefill_start", _i32p_t), ("prefill_len", _i32p_t),
                ("prefill_record_row", _i32p_t),
                ("num_preempted", ctypes.c_int32), ("preempted", _i64p_t),
                ("num_finished", ctypes.c_int32), ("finished", _i64p_t),
                ("num_released", ctypes.c_int32)]


class _CompressInfo(ctypes.Structure):
    _fields_ = [("units", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("resident_per_cu", ctypes.c_int32), ("compute_units", ctypes.c_int32),
                ("k_cached", ctypes.c_int32), ("wall_clock_khz", ctypes.c_int32)]


class _Debug(ctypes.Structure):
    _fields_ = [("importance", ctypes.c_void_p), ("redundancy", ctypes.c_void_p),
                ("score", ctypes.c_void_p), ("kept", ctypes.c_void_p),
                ("phase_times", ctypes.c_void_p)]


ZP_COMPRESS_KEEP_PREFIX = 1


class _DecodeArgs(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("num_reqs", ctypes.c_int32), ("q", ctypes.c_void_p),
                ("block_tables", ctypes.c_void_p), ("max_blocks", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("scale", ctypes.c_float), ("out", ctypes.c_void_p),
                ("out_dtype", ctypes.c_int32), ("lse_out", ctypes.c_void_p),
                ("q_out", ctypes.c_void_p), ("rows", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stream", ctypes.c_void_p)]


class _CompressArgs(ctypes.Structure):
    _fields_ = [("n_src", ctypes.c_int32), ("n_max", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_reqs", ctypes.c_int32), ("block_tables", ctypes.POINTER(ctypes.c_int32)),
                ("device_tables", ctypes.c_void_p), ("window_q", ctypes.POINTER(ctypes.c_void_p)),
                ("window_lse", ctypes.POINTER(ctypes.c_void_p)), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("freed_ids", ctypes.POINTER(ctypes.c_int32)),
                ("num_freed", ctypes.POINTER(ctypes.c_int32)), ("stream", ctypes.c_void_p),
                ("debug", ctypes.POINTER(_Debug)), ("flags", ctypes.c_uint32),
                ("num_blocks", ctypes.POINTER(ctypes.c_int32)), ("window_slots", ctypes.c_void_p),
                ("window_store_slots", ctypes.c_int32)]


_i32p = ctypes.POINTER(ctypes.c_int32)
_vp = ctypes.c_void_p
_lib = None


def lib() -> ctypes.CDLL:
    """Load libzp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__; __graft_entry__.build()')")
    # One HIP runtime per process: PyTorch ships its own libamdhip64, and
    # libzp.so binds to whichever copy is loaded first.  Loading torch first
    # makes it the same one; a second runtime loaded beside torch's sees no
    # device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    S = ctypes.c_int  # zp_status
    sig = {
        "zp_last_error": (ctypes.c_char_p, []),
        "zp_version": (ctypes.c_int32, []),
        "zp_block_pool_create": (S, [ctypes.c_int32, ctypes.c_uint32, ctypes.POINTER(_vp)]),
        "zp_block_pool_destroy": (None, [_vp]),
        "zp_block_alloc": (S, [_vp, ctypes.c_int32, _i32p]),
        "zp_block_share": (S, [_vp, _i32p, ctypes.c_int32]),
        "zp_block_release": (S, [_vp, _i32p, ctypes.c_int32, _i32p, _i32p]),
        "zp_block_refcount": (ctypes.c_int32, [_vp, ctypes.c_int32]),
        "zp_block_num_free": (ctypes.c_int32, [_vp]),
        "zp_block_num_pending": (ctypes.c_int32, [_vp]),
        "zp_block_pool_fence": (S, [_vp]),
        "zp_block_pool_sync": (S, [_vp]),
        "zp_compress_plan": (S, [_vp, ctypes.c_int32, ctypes.c_int32, _i32p, _i32p, _i32p, _i32p,
                                 _i32p]),
        "zp_compress_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_KVCache), ctypes.c_int32,
                                                          ctypes.c_int32, ctypes.c_int32]),
        "zp_compress": (S, [ctypes.POINTER(_KVCache), _vp, ctypes.c_int32, ctypes.c_int32,
                            ctypes.c_int32, _i32p, ctypes.POINTER(_vp), _vp, ctypes.c_size_t,
                            _i32p, _i32p, _vp, ctypes.POINTER(_Debug)]),
        "zp_compress_lse": (S, [ctypes.POINTER(_KVCache), _vp, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_int32, _i32p, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                _vp, ctypes.c_size_t, _i32p, _i32p, _vp,
                                ctypes.POINTER(_Debug)]),
        "zp_compress_n": (S, [ctypes.POINTER(_KVCache), _vp, ctypes.c_int32, ctypes.c_int32,
                              ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.POINTER(_vp),
                              ctypes.POINTER(_vp), _vp, ctypes.c_size_t, _i32p, _i32p, _vp,
                              ctypes.POINTER(_Debug)]),
        "zp_compress_keep_prefix": (S, [ctypes.POINTER(_KVCache), _vp, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                        ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp,
                                        ctypes.c_size_t, _i32p, _i32p, _vp,
                                        ctypes.POINTER(_Debug)]),
        "zp_compress_plan_n": (S, [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p,
                                   _i32p, _i32p, _i32p, _i32p]),
        "zp_compress_workspace_bytes_n": (ctypes.c_size_t, [ctypes.POINTER(_KVCache),
                                                            ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.c_int32, ctypes.c_int32]),
        "zp_compress_ex": (S, [ctypes.POINTER(_KVCache), _vp, ctypes.POINTER(_CompressArgs)]),
        "zp_compress_query": (S, [ctypes.POINTER(_KVCache), ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_CompressInfo)]),
        "zp_append_kv": (S, [ctypes.POINTER(_KVCache), ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                             _vp, _vp]),
        "zp_paged_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_KVCache),
                                                              ctypes.c_int32, ctypes.c_int32]),
        "zp_debug_flags": (ctypes.c_uint32, []),
        "zp_set_debug_flags": (S, [ctypes.c_uint32]),
        "zp_trace_available": (ctypes.c_int32, []),
        "zp_profile_enable": (S, [ctypes.c_int32]),
        "zp_profile_read": (S, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
        "zp_paged_decode": (S, [ctypes.POINTER(_KVCache), ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                                ctypes.c_int32, _vp, ctypes.c_float, _vp, _vp, ctypes.c_size_t,
                                _vp]),
        "zp_paged_decode_lse": (S, [ctypes.POINTER(_KVCache), ctypes.c_int32, ctypes.c_int32, _vp,
                                    _vp, ctypes.c_int32, _vp, ctypes.c_float, _vp, _vp, _vp, _vp,
                                    ctypes.c_int32, _vp, ctypes.c_size_t, _vp]),
        "zp_paged_decode_ex": (S, [ctypes.POINTER(_KVCache), ctypes.POINTER(_DecodeArgs)]),
        "zp_paged_decode_noalloc": (S, [ctypes.POINTER(_KVCache), ctypes.c_int32, ctypes.c_int32,
                                        _vp, _vp, ctypes.c_int32, _vp, ctypes.c_float, _vp, _vp,
                                        _vp, _vp, ctypes.c_int32, _vp]),
        "zp_redundancy_all": (S, [ctypes.POINTER(_KVCache), ctypes.c_int32, ctypes.c_int32, _vp,
                                  ctypes.c_int32, _vp, _vp]),
        "zp_prefix_index_create": (S, [_vp, ctypes.c_int32, ctypes.POINTER(_vp)]),
        "zp_prefix_index_destroy": (None, [_vp]),
        "zp_prefix_insert": (S, [_vp, _i32p, ctypes.c_int32, _i32p, ctypes.c_int32, _i32p]),
        "zp_prefix_match": (S, [_vp, _i32p, ctypes.c_int32, _i32p, _i32p]),
        "zp_prefix_evict": (S, [_vp, ctypes.c_int32, _i32p, _i32p]),
        "zp_prefix_size": (ctypes.c_int32, [_vp]),
        "zp_sched_create": (S, [_vp, ctypes.POINTER(_SchedConfig), ctypes.POINTER(_vp)]),
        "zp_sched_destroy": (None, [_vp]),
        "zp_sched_add": (S, [_vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
        "zp_sched_plan": (S, [_vp, ctypes.POINTER(_SchedStep)]),
        "zp_sched_tables": (S, [_vp, _i64p_t, ctypes.c_int32, ctypes.c_int32, _i32p, _i32p]),
        "zp_sched_compress_commit": (S, [_vp, _i32p]),
        "zp_sched_stats": (S, [_vp, _i32p, _i32p, _i32p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return lib().zp_last_error().decode()


def _check(status: int) -> None:
    if status != ZP_OK:
        raise ZpError(status, last_error())


def _i32(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_i32p)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _want(t, name: str, device, dtype, shape) -> None:
    """Raise ValueError unless ``t`` is a contiguous tensor on ``device`` with
    ``dtype`` and ``shape`` (None entries of ``shape`` match any size).  The
    kernels take raw pointers: a CPU tensor, a wrong element type or a short
    buffer would send them to invalid addresses, which the C layer cannot
    see."""
    if not hasattr(t, "data_ptr") or not hasattr(t, "is_contiguous"):
        raise ValueError(f"{name}: expected a tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, the cache is on {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None:
        got = tuple(int(x) for x in t.shape)
        if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
            want = tuple("*" if w is None else w for w in shape)
            raise ValueError(f"{name}: shape {got}, expected {want}")


def _want_bytes(t, name: str, device, nbytes: int) -> None:
    """A contiguous device buffer of at least ``nbytes`` bytes (workspaces)."""
    _want(t, name, device, None, None)
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, needs {nbytes}")


# --------------------------------------------------------------------------- pool

class BlockPool:
    """Host block pool (reference counts, free set, deferred frees)."""

    def __init__(self, num_blocks: int, manual_fence: bool = False):
        h = _vp()
        _check(lib().zp_block_pool_create(num_blocks, ZP_POOL_MANUAL_FENCE if manual_fence else 0,
                                          ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("pool destroyed")
        return self._h

    def close(self):
        if self._h is not None:
            lib().zp_block_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int) -> np.ndarray:
        ids = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib().zp_block_alloc(self.handle, n, _i32(ids)))
        return ids[:n]

    def share(self, ids: Sequence[int]) -> None:
        a = np.ascontiguousarray(ids, dtype=np.int32)
        _check(lib().zp_block_share(self.handle, _i32(a), int(a.size)))

    def release(self, ids: Sequence[int]) -> np.ndarray:
        a = np.ascontiguousarray(ids, dtype=np.int32)
        freed = np.zeros(max(a.size, 1), dtype=np.int32)
        n = np.zeros(1, dtype=np.int32)
        _check(lib().zp_block_release(self.handle, _i32(a), int(a.size), _i32(freed), _i32(n)))
        return freed[: int(n[0])]

    def refcount(self, i: int) -> int:
        return int(lib().zp_block_refcount(self.handle, i))

    def refcounts(self) -> np.ndarray:
        return np.array([self.refcount(i) for i in range(self.num_blocks)], dtype=np.int32)

    def num_free(self) -> int:
        return int(lib().zp_block_num_free(self.handle))

    def num_pending(self) -> int:
        return int(lib().zp_block_num_pending(self.handle))

    def fence(self) -> None:
        _check(lib().zp_block_pool_fence(self.handle))

    def sync(self) -> None:
        _check(lib().zp_block_pool_sync(self.handle))

    @classmethod
    def from_refcounts(cls, refcounts: np.ndarray, manual_fence: bool = False) -> "BlockPool":
        """A pool whose reference counts equal ``refcounts`` (allocate every
        referenced block, then share it up to its count)."""
        rc = np.asarray(refcounts, dtype=np.int32)
        pool = cls(int(rc.size), manual_fence=manual_fence)
        used = np.flatnonzero(rc > 0).astype(np.int32)
        if used.size:
            got = pool.alloc(int(rc.size))  # every id, smallest first
            unused = got[rc[got] == 0]
            if unused.size:
                pool.release(unused)
            extra = np.repeat(used, rc[used] - 1).astype(np.int32)
            if extra.size:
                pool.share(extra)
        return pool


def compress_plan(pool: BlockPool, n_max: int, tables: np.ndarray):
    """Host planner (zp_compress_plan, or zp_compress_plan_n when ``tables``,
    int32 [R][n_src], has more than n_max columns).  ``tables`` is rewritten
    in place; returns (src, dst, freed)."""
    assert tables.dtype == np.int32 and tables.flags.c_contiguous
    R, n_src = (int(x) for x in tables.shape)
    src = np.zeros((R, n_src), dtype=np.int32)
    dst = np.zeros((R, max(n_max - 1, 1)), dtype=np.int32)
    freed = np.zeros(max(R * n_src, 1), dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    if n_src == n_max:
        _check(lib().zp_compress_plan(pool.handle, n_max, R, _i32(tables), _i32(src), _i32(dst),
                                      _i32(freed), _i32(n)))
    else:
        _check(lib().zp_compress_plan_n(pool.handle, n_src, n_max, R, _i32(tables), _i32(src),
                                        _i32(dst), _i32(freed), _i32(n)))
    return src, dst, freed[: int(n[0])]


# --------------------------------------------------------------------------- cache

class KVCache:
    """Geometry plus per-layer K and V pools (caller-owned device tensors,
    each [num_blocks][num_kv_heads][block_size][head_dim])."""

    def __init__(self, k_pools: List, v_pools: List, num_q_heads: int):
        assert len(k_pools) == len(v_pools) and k_pools
        k0 = k_pools[0]
        nb, H, b, d = (int(x) for x in k0.shape)
        self.k_pools, self.v_pools = list(k_pools), list(v_pools)
        self.num_layers = len(k_pools)
        self.num_kv_heads, self.num_q_heads = H, int(num_q_heads)
        self.head_dim, self.block_size, self.num_blocks = d, b, nb
        name = str(k0.dtype)
        if name.endswith("bfloat16"):
            self.dtype = ZP_BF16
        elif name.endswith("float32"):
            self.dtype = ZP_F32
        else:
            raise ValueError(f"unsupported cache dtype {k0.dtype}")
        for t in self.k_pools + self.v_pools:
            if tuple(t.shape) != (nb, H, b, d) or t.dtype != k0.dtype or not t.is_contiguous():
                raise ValueError("every pool must be a contiguous tensor of the same shape and dtype")
        self.device = k0.device
        self.torch_dtype = k0.dtype
        if self.device.type != "cuda":
            raise ValueError(f"the pools must be GPU tensors, got {self.device}")
        if any(t.device != self.device for t in self.k_pools + self.v_pools):
            raise ValueError("every pool must be on the same device")
        n = self.num_layers
        self._k_arr = (_vp * n)(*[t.data_ptr() for t in self.k_pools])
        self._v_arr = (_vp * n)(*[t.data_ptr() for t in self.v_pools])
        self.c = _KVCache(n, H, self.num_q_heads, d, b, nb, self.dtype,
                          ctypes.cast(self._k_arr, ctypes.POINTER(_vp)),
                          ctypes.cast(self._v_arr, ctypes.POINTER(_vp)))

    @property
    def ref(self):
        return ctypes.byref(self.c)


def compress_workspace_bytes(cache: KVCache, num_reqs: int, n_max: int, window: int,
                             n_src: Optional[int] = None) -> int:
    if n_src is None or n_src == n_max:
        n = int(lib().zp_compress_workspace_bytes(cache.ref, num_reqs, n_max, window))
    else:
        n = int(lib().zp_compress_workspace_bytes_n(cache.ref, num_reqs, n_src, n_max, window))
    if n == 0:
        raise ZpError(ZP_ERR_INVALID, last_error())
    return n


def compress_query(cache: KVCache, num_reqs: int, n_max: int, window: int,
                   n_src: Optional[int] = None) -> dict:
    """zp_compress_query: how a compression call of this shape runs on the
    current device (units, threads, resident workgroups per compute unit,
    compute units, and whether the fused compaction loads K normally)."""
    info = _CompressInfo()
    _check(lib().zp_compress_query(cache.ref, num_reqs, n_max if n_src is None else n_src, n_max,
                                   window, ctypes.byref(info)))
    return {f: int(getattr(info, f)) for f, _ in _CompressInfo._fields_}


def compress(cache: KVCache, pool: BlockPool, n_max: int, window: int, tables: np.ndarray,
             window_q: List, workspace, stream=None, debug: Optional[dict] = None,
             window_lse: Optional[List] = None, keep_prefix: bool = False,
             device_tables=None, num_blocks=None, window_slots=None) -> np.ndarray:
    """zp_compress (zp_compress_lse when ``window_lse``, per-layer float
    tensors [R][w][Hq] of the window rows' normalisers, is given;
    zp_compress_n when ``tables`` has n_src > n_max columns).  ``tables``
    (host int32 [R][n_src]) is rewritten on success; returns the freed block
    ids.  ``keep_prefix``: zp_compress_keep_prefix (shared blocks the
    compaction leaves unchanged stay shared).  ``device_tables`` (device
    int32 [R][n_src], the same ids as ``tables``): zp_compress_ex with the
    caller's device copy, so an in-place plan uploads nothing.  ``num_blocks``
    (host int32 [R]): the blocks each request holds, its row padded with -1
    (zp_compress_ex: requests past the cap by different amounts in one
    call).  ``window_slots`` (device int32 [R]): zp_compress_ex reading the
    window rows in place from query-slot stores -- ``window_q[l]`` is then
    [S*w][Hq][d] and ``window_lse[l]`` [S*w][Hq], request r's rows those of
    slot window_slots[r]."""
    import torch
    if not (isinstance(tables, np.ndarray) and tables.dtype == np.int32 and tables.ndim == 2
            and tables.flags.c_contiguous):
        raise ValueError("tables: expected a C-contiguous host int32 [R][n_src] array")
    R, n_src = (int(x) for x in tables.shape)
    L, H, Hq, d, b = (cache.num_layers, cache.num_kv_heads, cache.num_q_heads, cache.head_dim,
                      cache.block_size)
    dev = cache.device
    if len(window_q) != L:
        raise ValueError(f"window_q: {len(window_q)} entries for {L} layers")
    S = 0
    if window_slots is not None:
        _want(window_slots, "window_slots", dev, torch.int32, (R,))
        rows = int(window_q[0].shape[0]) if len(window_q[0].shape) == 3 else -1
        if rows < window or rows % window:
            raise ValueError(f"window_q[0]: expected a query-slot store [S*{window}][Hq][d], "
                             f"got shape {tuple(window_q[0].shape)}")
        S = rows // window
    for l, t in enumerate(window_q):
        _want(t, f"window_q[{l}]", dev, cache.torch_dtype,
              (S * window, Hq, d) if S else (R, window, Hq, d))
    if window_lse is not None:
        if len(window_lse) != L:
            raise ValueError(f"window_lse: {len(window_lse)} entries for {L} layers")
        for l, t in enumerate(window_lse):
            _want(t, f"window_lse[{l}]", dev, torch.float32,
                  (S * window, Hq) if S else (R, window, Hq))
    _want(workspace, "workspace", dev, None, None)
    if device_tables is not None:
        _want(device_tables, "device_tables", dev, torch.int32, (R, n_src))
    if debug:
        T, k_keep = n_src * b, (n_max - 1) * b
        for key in ("importance", "redundancy", "score"):
            if debug.get(key) is not None:
                _want(debug[key], f"debug[{key!r}]", dev, torch.float32, (L, R, H, T))
        if debug.get("kept") is not None:
            _want(debug["kept"], "debug['kept']", dev, torch.int32, (L, R, H, k_keep))
        if debug.get("phase_times") is not None:
            _want(debug["phase_times"], "debug['phase_times']", dev, torch.int64, (L, R, H, 5))
    wq = (_vp * cache.num_layers)(*[t.data_ptr() for t in window_q])
    wl = None
    if window_lse is not None:
        wl = (_vp * cache.num_layers)(*[t.data_ptr() for t in window_lse])
    freed = np.zeros(max(R * n_src, 1), dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    dbg = None
    if debug:
        dbg = _Debug(_dptr(debug.get("importance")), _dptr(debug.get("redundancy")),
                     _dptr(debug.get("score")), _dptr(debug.get("kept")),
                     _dptr(debug.get("phase_times")))
    nbk = None
    if num_blocks is not None:
        nbk = np.ascontiguousarray(num_blocks, dtype=np.int32)
        if nbk.shape != (R,):
            raise ValueError(f"num_blocks: shape {nbk.shape}, expected ({R},)")
    if device_tables is not None or nbk is not None or window_slots is not None:
        a = _CompressArgs(n_src, n_max, window, R, _i32(tables),
                          device_tables.data_ptr() if device_tables is not None else None,
                          ctypes.cast(wq, ctypes.POINTER(_vp)),
                          ctypes.cast(wl, ctypes.POINTER(_vp)) if wl is not None else None,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _i32(freed), _i32(n), _stream_handle(stream),
                          ctypes.pointer(dbg) if dbg else None,
                          ZP_COMPRESS_KEEP_PREFIX if keep_prefix else 0,
                          _i32(nbk) if nbk is not None else None,
                          window_slots.data_ptr() if window_slots is not None else None, S)
        st = lib().zp_compress_ex(cache.ref, pool.handle, ctypes.byref(a))
    elif keep_prefix:
        st = lib().zp_compress_keep_prefix(
            cache.ref, pool.handle, n_src, n_max, window, R, _i32(tables),
            ctypes.cast(wq, ctypes.POINTER(_vp)),
            ctypes.cast(wl, ctypes.POINTER(_vp)) if wl is not None else None,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), _i32(freed),
            _i32(n), _stream_handle(stream), ctypes.byref(dbg) if dbg else None)
    elif n_src != n_max:
        st = lib().zp_compress_n(cache.ref, pool.handle, n_src, n_max, window, R, _i32(tables),
                                 ctypes.cast(wq, ctypes.POINTER(_vp)),
                                 ctypes.cast(wl, ctypes.POINTER(_vp)) if wl is not None else None,
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                 _i32(freed), _i32(n), _stream_handle(stream),
                                 ctypes.byref(dbg) if dbg else None)
    elif wl is None:
        st = lib().zp_compress(cache.ref, pool.handle, n_max, window, R, _i32(tables),
                               ctypes.cast(wq, ctypes.POINTER(_vp)), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _i32(freed), _i32(n),
                               _stream_handle(stream), ctypes.byref(dbg) if dbg else None)
    else:
        st = lib().zp_compress_lse(cache.ref, pool.handle, n_max, window, R, _i32(tables),
                                   ctypes.cast(wq, ctypes.POINTER(_vp)),
                                   ctypes.cast(wl, ctypes.POINTER(_vp)), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _i32(freed),
                                   _i32(n), _stream_handle(stream),
                                   ctypes.byref(dbg) if dbg else None)
    _check(st)
    return freed[: int(n[0])]


def append_kv(cache: KVCache, layer: int, k_new, v_new, slot_mapping, stream=None) -> None:
    """zp_append_kv: k_new, v_new [R][H][d] (cache dtype), slot_mapping int32 [R]."""
    import torch
    dev = cache.device
    _want(slot_mapping, "slot_mapping", dev, torch.int32, (None,))
    kv = (int(slot_mapping.shape[0]), cache.num_kv_heads, cache.head_dim)
    _want(k_new, "k_new", dev, cache.torch_dtype, kv)
    _want(v_new, "v_new", dev, cache.torch_dtype, kv)
    _check(lib().zp_append_kv(cache.ref, layer, int(slot_mapping.shape[0]), k_new.data_ptr(),
                              v_new.data_ptr(), slot_mapping.data_ptr(), _stream_handle(stream)))


def paged_decode_workspace_bytes(cache: KVCache, num_reqs: int, max_blocks: int) -> int:
    return int(lib().zp_paged_decode_workspace_bytes(cache.ref, num_reqs, max_blocks))


def paged_decode(cache: KVCache, layer: int, q, tables, seq_lens, scale: float, out, workspace,
                 stream=None, lse_out=None, lse_rows=None, q_out=None) -> None:
    """zp_paged_decode, or zp_paged_decode_lse when ``lse_out`` (float
    [rows][Hq]) or ``q_out`` ([rows][Hq][d], cache dtype) is given;
    ``lse_rows`` (int32 [R]) maps requests to rows.  A bfloat16 ``out`` goes
    through zp_paged_decode_ex with out_dtype ZP_BF16."""
    import torch
    dev, Hq, d = cache.device, cache.num_q_heads, cache.head_dim
    _want(tables, "tables", dev, torch.int32, (None, None))
    R, max_blocks = (int(x) for x in tables.shape)
    _want(q, "q", dev, cache.torch_dtype, (R, Hq, d))
    _want(seq_lens, "seq_lens", dev, torch.int32, (R,))
    out_bf16 = hasattr(out, "dtype") and out.dtype == torch.bfloat16
    _want(out, "out", dev, torch.bfloat16 if out_bf16 else torch.float32, (R, Hq, d))
    if workspace is not None:
        _want(workspace, "workspace", dev, None, None)
    if lse_out is not None:
        _want(lse_out, "lse_out", dev, torch.float32, (None, Hq))
    if q_out is not None:
        _want(q_out, "q_out", dev, cache.torch_dtype, (None, Hq, d))
        if lse_out is not None and int(q_out.shape[0]) != int(lse_out.shape[0]):
            raise ValueError("q_out and lse_out must have the same number of rows")
    if lse_rows is not None:
        _want(lse_rows, "lse_rows", dev, torch.int32, (R,))
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if out_bf16:
        rows_src = lse_out if lse_out is not None else q_out
        a = _DecodeArgs(layer, R, q.data_ptr(), tables.data_ptr(), max_blocks, seq_lens.data_ptr(),
                        float(scale), out.data_ptr(), ZP_BF16, _dptr(lse_out), _dptr(q_out),
                        _dptr(lse_rows), int(rows_src.shape[0]) if rows_src is not None else 0,
                        ws_ptr, ws_bytes, _stream_handle(stream))
        _check(lib().zp_paged_decode_ex(cache.ref, ctypes.byref(a)))
        return
    if lse_out is None and q_out is None:
        _check(lib().zp_paged_decode(cache.ref, layer, R, q.data_ptr(), tables.data_ptr(),
                                     max_blocks, seq_lens.data_ptr(), float(scale), out.data_ptr(),
                                     ws_ptr, ws_bytes, _stream_handle(stream)))
        return
    cap = int((lse_out if lse_out is not None else q_out).shape[0])
    _check(lib().zp_paged_decode_lse(cache.ref, layer, R, q.data_ptr(), tables.data_ptr(),
                                     max_blocks, seq_lens.data_ptr(), float(scale), out.data_ptr(),
                                     _dptr(lse_out), _dptr(q_out), _dptr(lse_rows), cap,
                                     ws_ptr, ws_bytes, _stream_handle(stream)))


def paged_decode_noalloc(cache: KVCache, layer: int, q, tables, seq_lens, scale: float, out,
                         stream=None, lse_out=None, lse_rows=None, q_out=None) -> None:
    """zp_paged_decode_noalloc: paged_decode with the split partials in the
    library's fixed device scratch (no workspace; nothing is allocated).
    Calls whose work overlaps on one GPU race on that scratch."""
    import torch
    dev, Hq, d = cache.device, cache.num_q_heads, cache.head_dim
    _want(tables, "tables", dev, torch.int32, (None, None))
    R, max_blocks = (int(x) for x in tables.shape)
    _want(q, "q", dev, cache.torch_dtype, (R, Hq, d))
    _want(seq_lens, "seq_lens", dev, torch.int32, (R,))
    _want(out, "out", dev, torch.float32, (R, Hq, d))
    if lse_out is not None:
        _want(lse_out, "lse_out", dev, torch.float32, (None, Hq))
    if q_out is not None:
        _want(q_out, "q_out", dev, cache.torch_dtype, (None, Hq, d))
        if lse_out is not None and int(q_out.shape[0]) != int(lse_out.shape[0]):
            raise ValueError("q_out and lse_out must have the same number of rows")
    if lse_rows is not None:
        _want(lse_rows, "lse_rows", dev, torch.int32, (R,))
    rows_src = lse_out if lse_out is not None else q_out
    cap = int(rows_src.shape[0]) if rows_src is not None else 0
    _check(lib().zp_paged_decode_noalloc(cache.ref, layer, R, q.data_ptr(), tables.data_ptr(),
                                         max_blocks, seq_lens.data_ptr(), float(scale),
                                         out.data_ptr(), _dptr(lse_out), _dptr(q_out),
                                         _dptr(lse_rows), cap, _stream_handle(stream)))


def redundancy_all(cache: KVCache, layer: int, tables, out, stream=None) -> None:
    """zp_redundancy_all: tables device int32 [R][n_blocks], out float [R][H][T]."""
    import torch
    _want(tables, "tables", cache.device, torch.int32, (None, None))
    R, n_blocks = (int(x) for x in tables.shape)
    _want(out, "out", cache.device, torch.float32, (R, cache.num_kv_heads, n_blocks * cache.block_size))
    _check(lib().zp_redundancy_all(cache.ref, layer, R, tables.data_ptr(), n_blocks,
                                   out.data_ptr(), _stream_handle(stream)))


# --------------------------------------------------------------------------- prefix index

class PrefixIndex:
    """Prefix index (zp_prefix_*): full prompt blocks found again by tokens."""

    def __init__(self, pool: BlockPool, block_size: int):
        self.pool = pool
        self.block_size = block_size
        h = _vp()
        _check(lib().zp_prefix_index_create(pool.handle, block_size, ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.zp_prefix_index_destroy(self.handle)
            self.handle = None

    def insert(self, tokens, block_ids) -> int:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        ids = np.ascontiguousarray(block_ids, dtype=np.int32)
        n = np.zeros(1, dtype=np.int32)
        _check(lib().zp_prefix_insert(self.handle, _i32(t) if t.size else None, int(t.size),
                                      _i32(ids) if ids.size else None, int(ids.size), _i32(n)))
        return int(n[0])

    def match(self, tokens) -> np.ndarray:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        out = np.zeros(max(t.size // self.block_size, 1), dtype=np.int32)
        n = np.zeros(1, dtype=np.int32)
        _check(lib().zp_prefix_match(self.handle, _i32(t) if t.size else None, int(t.size),
                                     _i32(out), _i32(n)))
        return out[: int(n[0])].copy()

    def evict(self, max_entries: int) -> np.ndarray:
        out = np.zeros(max(max_entries, 1), dtype=np.int32)
        n = np.zeros(1, dtype=np.int32)
        _check(lib().zp_prefix_evict(self.handle, int(max_entries), _i32(out), _i32(n)))
        return out[: int(n[0])].copy()

    def __len__(self) -> int:
        return int(lib().zp_prefix_size(self.handle))


# --------------------------------------------------------------------------- scheduler

class Scheduler:
    """Hybrid scheduler (zp_sched_*): query slots only for requests in their
    observation window, preemption of slot-less requests first."""

    def __init__(self, pool: BlockPool, n_max: int, block_size: int, window: int,
                 num_query_slots: int, max_running: int, prefill_chunk: int = 0):
        self.pool = pool  # keeps the pool alive
        self.n_max, self.block_size, self.window = n_max, block_size, window
        self.prefill_chunk = prefill_chunk
        cfg = _SchedConfig(n_max, block_size, window, num_query_slots, max_running, prefill_chunk)
        h = _vp()
        _check(lib().zp_sched_create(pool.handle, ctypes.byref(cfg), ctypes.byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.zp_sched_destroy(self.handle)
            self.handle = None

    def add(self, req_id: int, prompt_len: int, max_new_tokens: int) -> None:
        _check(lib().zp_sched_add(self.handle, int(req_id), int(prompt_len), int(max_new_tokens)))

    def plan(self) -> dict:
        st = _SchedStep()
        _check(lib().zp_sched_plan(self.handle, ctypes.byref(st)))

        def arr(ptr, n, dt):
            return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dt).copy() if n else np.zeros(0, dt)
        return {
            "admitted": arr(st.admitted, st.num_admitted, np.int64),
            "decode_ids": arr(st.decode_ids, st.num_decode, np.int64),
            "decode_slot": arr(st.decode_slot, st.num_decode, np.int32),
            "decode_seq_len": arr(st.decode_seq_len, st.num_decode, np.int32),
            "decode_record_row": arr(st.decode_record_row, st.num_decode, np.int32),
            "compress_ids": arr(st.compress_ids, st.num_compress, np.int64),
            "compress_qslot": arr(st.compress_qslot, st.num_compress, np.int32),
            "compress_n_src": arr(st.compress_n_src, st.num_compress, np.int32),
            "prefill_ids": arr(st.prefill_ids, st.num_prefill, np.int64),
            "prefill_start": arr(st.prefill_start, st.num_prefill, np.int32),
            "prefill_len": arr(st.prefill_len, st.num_prefill, np.int32),
            "prefill_record_row": arr(st.prefill_record_row, st.num_prefill, np.int32),
            "preempted": arr(st.preempted, st.num_preempted, np.int64),
            "finished": arr(st.finished, st.num_finished, np.int64),
            "num_released": int(st.num_released),
        }

    def tables(self, ids, width: Optional[int] = None):
        ids = np.ascontiguousarray(ids, dtype=np.int64)
        width = self.n_max if width is None else int(width)
        tab = np.zeros((ids.size, width), dtype=np.int32)
        lens = np.zeros(max(ids.size, 1), dtype=np.int32)
        _check(lib().zp_sched_tables(self.handle, ids.ctypes.data_as(_i64p_t), int(ids.size), width,
                                     _i32(tab) if ids.size else None, _i32(lens)))
        return tab, lens[: ids.size]

    def compress_commit(self, new_tables: np.ndarray) -> None:
        t = np.ascontiguousarray(new_tables, dtype=np.int32)
        _check(lib().zp_sched_compress_commit(self.handle, _i32(t) if t.size else None))

    def stats(self) -> dict:
        w, r, f = (np.zeros(1, dtype=np.int32) for _ in range(3))
        _check(lib().zp_sched_stats(self.handle, _i32(w), _i32(r), _i32(f)))
        return {"waiting": int(w[0]), "running": int(r[0]), "free_query_slots": int(f[0])}


# --------------------------------------------------------------------------- debug switches

ZP_DEBUG_TRACE, ZP_DEBUG_POISON, ZP_DEBUG_VALIDATE = 1, 2, 4


def debug_flags() -> int:
    """The debug switches in effect (ZP_DEBUG_* bits)."""
    return int(lib().zp_debug_flags())


def set_debug_flags(flags: int) -> None:
    _check(lib().zp_set_debug_flags(int(flags)))


def trace_available() -> bool:
    return bool(lib().zp_trace_available())


# --------------------------------------------------------------------------- timing

PHASES = ("upload", "score_stats", "score", "select", "compact", "append", "decode", "combine",
          "redundancy_all", "score_compact")


def profile_enable(on: bool = True) -> None:
    _check(lib().zp_profile_enable(1 if on else 0))


def profile_read() -> dict:
    """{phase: (total_ms, launches)} accumulated since the last read."""
    ms = (ctypes.c_double * len(PHASES))()
    n = (ctypes.c_int64 * len(PHASES))()
    _check(lib().zp_profile_read(ms, n))
    return {p: (float(ms[i]), int(n[i])) for i, p in enumerate(PHASES)}
