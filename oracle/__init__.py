"""CPU oracle for Compressed PagedAttention (compression pass + paged decode).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.

The arithmetic lives in ``zp_oracle.c`` (plain C, double precision, OpenMP
over independent units).  This module only marshals NumPy arrays into it and
strings the steps together in the pages' order: plan the target blocks,
score every cached slot (observation-window importance and Lightning
Redundancy Score), select the survivors per (layer, head), compact them in
order into the first N_max-1 blocks, then append the pending token and run
dense decode attention.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from . import build as _build

_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ZP_ORACLE_LIBRARY")  # an instrumented build (sanitizer test)
    if not path:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    lib = ctypes.CDLL(path)
    lib.zpo_num_threads.restype = ctypes.c_int
    lib.zpo_plan.restype = ctypes.c_int
    lib.zpo_plan.argtypes = [ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p,
                             ctypes.c_int32, _i32p]
    lib.zpo_scores.restype = None
    lib.zpo_scores.argtypes = [ctypes.c_int32] * 8 + [ctypes.c_void_p, ctypes.c_void_p, _i32p,
                                                      _f64p, _f64p, _f64p]
    lib.zpo_select.restype = None
    lib.zpo_select.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                               _f64p, _i32p]
    lib.zpo_compact.restype = None
    lib.zpo_compact.argtypes = [ctypes.c_int64] + [ctypes.c_int32] * 8 + [
        ctypes.c_void_p, ctypes.c_void_p, _i32p, _i32p, _i32p]
    lib.zpo_append.restype = None
    lib.zpo_append.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_void_p] * 4 + [_i32p]
    lib.zpo_decode.restype = None
    lib.zpo_decode.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_void_p] * 3 + [
        _i32p, ctypes.c_int32, _i32p, ctypes.c_double, _f64p]
    lib.zpo_decode_lse.restype = None
    lib.zpo_decode_lse.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_void_p] * 2 + [
        _i32p, ctypes.c_int32, _i32p, ctypes.c_double, _f64p]
    lib.zpo_redundancy_all.restype = None
    lib.zpo_redundancy_all.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_void_p, _i32p, _f64p]
    _lib = lib
    return lib


def _i32(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_i32p)


def _f64(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_f64p)


def _vp(a: np.ndarray):
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


def num_threads() -> int:
    return int(_load().zpo_num_threads())


OK, INVALID, NO_BLOCKS = 0, 1, 2


@dataclass
class Plan:
    status: int
    tables: np.ndarray      # new tables [R][n_src]: n_max ids, then -1 for the surplus
    refcounts: np.ndarray   # new refcounts
    src: np.ndarray         # [R][n_src] (the old tables)
    dst: np.ndarray         # [R][n_max-1]
    freed: np.ndarray       # freed ids in order


def plan(refcounts: np.ndarray, tables: np.ndarray, n_max: int,
         first_evict: Optional[np.ndarray] = None, block_size: int = 0,
         n_blocks: Optional[np.ndarray] = None) -> Plan:
    """Target-block plan of one compression call (inputs are not modified).
    ``tables`` is [R][n_src] with n_src >= n_max.  ``first_evict`` ([R], the
    lowest evicted slot of each request over its layers and heads) keeps the
    shared blocks wholly below it shared.  ``n_blocks`` ([R]): request r holds
    only the first n_blocks[r] entries of its row, the rest being -1."""
    lib = _load()
    rc = np.ascontiguousarray(refcounts, dtype=np.int32).copy()
    tab = np.ascontiguousarray(tables, dtype=np.int32).copy()
    R, n_src = (int(x) for x in tab.shape)
    src = np.zeros((R, n_src), dtype=np.int32)
    dst = np.zeros((R, max(n_max - 1, 1)), dtype=np.int32)
    freed = np.zeros(max(R * n_src, 1), dtype=np.int32)
    nfreed = np.zeros(1, dtype=np.int32)
    fe = nb = None
    if first_evict is not None:
        fe_a = np.ascontiguousarray(first_evict, dtype=np.int32)
        fe = _i32(fe_a)
    if n_blocks is not None:
        nb_a = np.ascontiguousarray(n_blocks, dtype=np.int32)
        nb = _i32(nb_a)
    st = lib.zpo_plan(int(rc.shape[0]), _i32(rc), R, n_src, n_max, _i32(tab), _i32(src),
                      _i32(dst), _i32(freed), _i32(nfreed), fe, int(block_size), nb)
    return Plan(int(st), tab, rc, src, dst, freed[: int(nfreed[0])].copy())


def scores(kpool: np.ndarray, window_q: np.ndarray, src: np.ndarray, *, num_kv_heads: int,
           num_q_heads: int, head_dim: int, block_size: int, window: int,
           n_max: Optional[int] = None):
    """Importance A, redundancy R and combined score s, each [R][H][T] float64,
    over the T = n_src*b slots of the tables ``src`` [R][n_src] (``n_max``,
    if given, must be that block count)."""
    lib = _load()
    is_bf16 = int(kpool.dtype == np.uint16)
    R, n_src = (int(x) for x in src.shape)
    assert n_max is None or n_max == n_src
    T = n_src * block_size
    A = np.zeros((R, num_kv_heads, T))
    Rr = np.zeros((R, num_kv_heads, T))
    s = np.zeros((R, num_kv_heads, T))
    lib.zpo_scores(num_kv_heads, num_q_heads, head_dim, block_size, is_bf16, n_src, window, R,
                   _vp(np.ascontiguousarray(kpool)), _vp(np.ascontiguousarray(window_q)),
                   _i32(np.ascontiguousarray(src, dtype=np.int32)), _f64(A), _f64(Rr), _f64(s))
    return A, Rr, s


def select(s: np.ndarray, window: int, k_sel: int) -> np.ndarray:
    """Ascending kept slots per unit: s [..., T] float64 -> int32 [..., k_sel + w]."""
    lib = _load()
    T = int(s.shape[-1])
    lead = s.shape[:-1]
    flat = np.ascontiguousarray(s.reshape(-1, T), dtype=np.float64)
    kept = np.zeros((flat.shape[0], k_sel + window), dtype=np.int32)
    lib.zpo_select(int(flat.shape[0]), T, window, k_sel, _f64(flat), _i32(kept))
    return kept.reshape(*lead, k_sel + window)


def compact(pool: np.ndarray, src: np.ndarray, dst: np.ndarray, kept: np.ndarray, *,
            n_max: int) -> np.ndarray:
    """Out-of-place order-preserving compaction of one [nb][H][b][d] pool
    (src [R][n_src] old tables, dst [R][n_max-1] targets)."""
    lib = _load()
    pool = np.ascontiguousarray(pool)
    nb, H, b, d = pool.shape
    out = np.empty_like(pool)
    R, n_src = (int(x) for x in src.shape)
    k_keep = int(kept.shape[-1])
    lib.zpo_compact(int(pool.size), H, d, b, pool.itemsize, n_src, n_max, R, k_keep, _vp(pool),
                    _vp(out),
                    _i32(np.ascontiguousarray(src, dtype=np.int32)),
                    _i32(np.ascontiguousarray(dst, dtype=np.int32)),
                    _i32(np.ascontiguousarray(kept, dtype=np.int32)))
    return out


def append(kpool: np.ndarray, vpool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
           slot_mapping: np.ndarray) -> None:
    """In-place append of one token per request into the pools (host copies)."""
    lib = _load()
    nb, H, b, d = kpool.shape
    R = int(slot_mapping.shape[0])
    lib.zpo_append(H, d, b, kpool.itemsize, R, _vp(kpool), _vp(vpool),
                   _vp(np.ascontiguousarray(k_new)), _vp(np.ascontiguousarray(v_new)),
                   _i32(np.ascontiguousarray(slot_mapping, dtype=np.int32)))


def decode(kpool: np.ndarray, vpool: np.ndarray, q: np.ndarray, tables: np.ndarray,
           seq_lens: np.ndarray, *, num_q_heads: int, scale: Optional[float] = None) -> np.ndarray:
    """Dense paged decode attention in double: [R][Hq][d] float64."""
    lib = _load()
    nb, H, b, d = kpool.shape
    is_bf16 = int(kpool.dtype == np.uint16)
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    R, max_blocks = tables.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((R, num_q_heads, d))
    lib.zpo_decode(H, num_q_heads, d, b, is_bf16, R, _vp(np.ascontiguousarray(kpool)),
                   _vp(np.ascontiguousarray(vpool)), _vp(np.ascontiguousarray(q)), _i32(tables),
                   max_blocks, _i32(np.ascontiguousarray(seq_lens, dtype=np.int32)), float(scale),
                   _f64(out))
    return out


def decode_lse(kpool: np.ndarray, q: np.ndarray, tables: np.ndarray, seq_lens: np.ndarray, *,
               num_q_heads: int, scale: Optional[float] = None) -> np.ndarray:
    """log sum_j exp(scale q.k_j) over each request's slots, in double: [R][Hq]."""
    lib = _load()
    nb, H, b, d = kpool.shape
    is_bf16 = int(kpool.dtype == np.uint16)
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    R, max_blocks = tables.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((R, num_q_heads))
    lib.zpo_decode_lse(H, num_q_heads, d, b, is_bf16, R, _vp(np.ascontiguousarray(kpool)),
                       _vp(np.ascontiguousarray(q)), _i32(tables), max_blocks,
                       _i32(np.ascontiguousarray(seq_lens, dtype=np.int32)), float(scale),
                       _f64(out))
    return out


def window_lse(kpool: np.ndarray, window_q: np.ndarray, tables: np.ndarray, *, n_max: int,
               window: int, num_q_heads: int) -> np.ndarray:
    """Normalisers of the window rows: for window position i, the log-sum-exp
    of q_i.k_j/sqrt(d) over slots j <= T-w+i (causal window): [R][w][Hq]."""
    b = kpool.shape[2]
    T = n_max * b
    R = tables.shape[0]
    out = np.zeros((R, window, num_q_heads))
    for i in range(window):
        lens = np.full(R, T - window + i + 1, dtype=np.int32)
        out[:, i, :] = decode_lse(kpool, np.ascontiguousarray(window_q[:, i]), tables, lens,
                                  num_q_heads=num_q_heads)
    return out


def redundancy_all(kpool: np.ndarray, tables: np.ndarray) -> np.ndarray:
    """All-pairs redundancy (mean cosine with every other slot of the
    sequence) over the T = n_blocks*b slots of each table row: [R][H][T]."""
    lib = _load()
    nb, H, b, d = kpool.shape
    is_bf16 = int(kpool.dtype == np.uint16)
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    R, n_blocks = tables.shape
    out = np.zeros((R, H, n_blocks * b))
    lib.zpo_redundancy_all(H, d, b, is_bf16, n_blocks, R, _vp(np.ascontiguousarray(kpool)),
                           _i32(tables), _f64(out))
    return out


@dataclass
class CompressResult:
    plan: Plan
    A: List[np.ndarray]       # per layer [R][H][T]
    R: List[np.ndarray]
    s: List[np.ndarray]
    kept: List[np.ndarray]    # per layer [R][H][K_keep]
    k_pool: List[np.ndarray]  # compacted pools (out of place)
    v_pool: List[np.ndarray]


def first_evicted(kept: List[np.ndarray], T, window: int) -> np.ndarray:
    """Lowest evicted slot of each request over all layers and heads, from
    the kept lists ([R][H][K_keep] per layer); ``T`` is the cached slots of
    every request, or an array of them per request."""
    R = kept[0].shape[0]
    Ts = np.broadcast_to(np.asarray(T, dtype=np.int64), (R,))
    Tm = int(Ts.max())
    C = Ts - window
    out = None
    for k in kept:
        mask = np.ones(k.shape[:2] + (Tm,), dtype=bool)
        np.put_along_axis(mask, k.astype(np.int64), False, axis=-1)
        mask &= np.arange(Tm)[None, None, :] < C[:, None, None]
        first = np.where(mask.any(-1), mask.argmax(-1), C[:, None]).min(axis=1)
        out = first if out is None else np.minimum(out, first)
    return out.astype(np.int32)


def _compress_ragged(case, layers, with_pools, keep_prefix) -> "CompressResult":
    """compress() for requests holding different numbers of blocks
    (``case.num_blocks``): one plan for the whole call, then every request on
    its own T = num_blocks[r]*b (scores and selection are per (request,
    head) anyway); the compaction writes only each request's own targets, so
    the per-request results merge without overlap.  A, R and s come back
    padded to the longest T with NaN."""
    g = case.geom
    n_max, w, b = case.n_max, case.window, g.block_size
    k_sel = (n_max - 1) * b - w
    nbk = np.asarray(case.num_blocks, dtype=np.int32)
    R, Tm = case.num_reqs, int(nbk.max()) * b
    layers = list(range(g.num_layers)) if layers is None else layers
    kw = dict(num_kv_heads=g.num_kv_heads, num_q_heads=g.num_q_heads, head_dim=g.head_dim,
              block_size=b, window=w)

    def unit_scores(layer, src):
        A = np.full((R, g.num_kv_heads, Tm), np.nan)
        Rr, s = A.copy(), A.copy()
        kept = np.zeros((R, g.num_kv_heads, (n_max - 1) * b), dtype=np.int32)
        for r in range(R):
            n = int(nbk[r])
            a, rr, ss = scores(case.k_pool[layer], case.window_q[layer][r:r + 1],
                               np.ascontiguousarray(src[r:r + 1, :n]), **kw)
            A[r, :, :n * b], Rr[r, :, :n * b], s[r, :, :n * b] = a[0], rr[0], ss[0]
            kept[r] = select(ss[0], w, k_sel)
        return A, Rr, s, kept

    sel = {}
    if keep_prefix:
        for layer in range(g.num_layers):
            sel[layer] = unit_scores(layer, case.tables)
        fe = first_evicted([sel[l][3] for l in range(g.num_layers)], nbk * b, w)
        p = plan(case.refcounts, case.tables, n_max, fe, b, n_blocks=nbk)
    else:
        p = plan(case.refcounts, case.tables, n_max, n_blocks=nbk)
    if p.status != OK:
        raise RuntimeError(f"oracle plan failed with status {p.status}")
    out = CompressResult(p, [], [], [], [], [], [])
    for layer in layers:
        A, Rr, s, kept = sel[layer] if layer in sel else unit_scores(layer, p.src)
        out.A.append(A)
        out.R.append(Rr)
        out.s.append(s)
        out.kept.append(kept)
        if with_pools:
            for pools, res in ((case.k_pool, out.k_pool), (case.v_pool, out.v_pool)):
                merged = pools[layer].copy()
                for r in range(R):
                    n = int(nbk[r])
                    one = compact(pools[layer], np.ascontiguousarray(p.src[r:r + 1, :n]),
                                  p.dst[r:r + 1], kept[r:r + 1], n_max=n_max)
                    merged[p.dst[r]] = one[p.dst[r]]
                res.append(merged)
    return out


def compress(case, layers: Optional[List[int]] = None, with_pools: bool = True,
             keep_prefix: bool = False) -> CompressResult:
    """The whole compression call of a synthetic case, step by step
    (``with_pools=False`` skips the out-of-place compaction of the pools).
    ``keep_prefix``: the plan is made after the selection of every layer, and
    shared blocks below each request's first eviction stay shared."""
    if getattr(case, "num_blocks", None) is not None:
        return _compress_ragged(case, layers, with_pools, keep_prefix)
    g = case.geom
    n_max, w, b = case.n_max, case.window, g.block_size
    k_keep = (n_max - 1) * b
    k_sel = k_keep - w
    T = case.tables.shape[1] * b
    layers = list(range(g.num_layers)) if layers is None else layers
    sel = {}
    if keep_prefix:
        for layer in range(g.num_layers):
            A, Rr, s = scores(case.k_pool[layer], case.window_q[layer], case.tables,
                              num_kv_heads=g.num_kv_heads, num_q_heads=g.num_q_heads,
                              head_dim=g.head_dim, block_size=b, window=w)
            sel[layer] = (A, Rr, s, select(s, w, k_sel))
        fe = first_evicted([sel[l][3] for l in range(g.num_layers)], T, w)
        p = plan(case.refcounts, case.tables, n_max, fe, b)
    else:
        p = plan(case.refcounts, case.tables, n_max)
    if p.status != OK:
        raise RuntimeError(f"oracle plan failed with status {p.status}")
    out = CompressResult(p, [], [], [], [], [], [])
    for layer in layers:
        if layer in sel:
            A, Rr, s, kept = sel[layer]
        else:
            A, Rr, s = scores(case.k_pool[layer], case.window_q[layer], p.src,
                              num_kv_heads=g.num_kv_heads, num_q_heads=g.num_q_heads,
                              head_dim=g.head_dim, block_size=b, window=w)
            kept = select(s, w, k_sel)
        out.A.append(A)
        out.R.append(Rr)
        out.s.append(s)
        out.kept.append(kept)
        if with_pools:
            out.k_pool.append(compact(case.k_pool[layer], p.src, p.dst, kept, n_max=n_max))
            out.v_pool.append(compact(case.v_pool[layer], p.src, p.dst, kept, n_max=n_max))
    return out
