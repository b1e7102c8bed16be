"""Seeded synthetic inputs for the compression pass and paged decode.

This module only draws random numbers and lays them out. It holds none of
the method's arithmetic (no scores, no selection, no attention), so that the
CPU oracle and the HIP path can both be fed from it without sharing code.

Recipe (all NumPy ``default_rng(seed)``, PCG64):
  * physical block ids: ``rng.permutation(pool)``; request r takes ids
    ``perm[r*n_max:(r+1)*n_max]`` in order (shared-prefix cases take the
    prefix ids first);
  * values: float64 standard normals -> float32 -> bfloat16 by round to
    nearest even on the bit pattern (bf16 caches) or kept float32;
  * pool blocks that no request references are filled with NaN, so a stray
    read shows up in every comparison.

Shapes follow the paged KV layout used throughout: one K and one V pool per
layer, ``[num_blocks][H][b][d]``; window queries ``[R][w][Hq][d]``; pending
decode token ``q [R][Hq][d]``, ``k, v [R][H][d]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Finite inputs cannot overflow the 32-bit sum (the largest finite pattern
    plus 0x8000 stays below 2^32); NaNs are mapped to a quiet bf16 NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    rounded = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = BF16_NAN
    return rounded


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Geometry:
    num_layers: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    dtype: str  # "f32" or "bf16"

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.uint16


@dataclass
class CompressCase:
    """One compression call followed by one decode step.

    ``k_pool[l]`` / ``v_pool[l]`` are the physical pools of layer l, stored as
    float32 (dtype "f32") or bfloat16 bit patterns (dtype "bf16").
    ``refcounts`` counts table references plus any ``extra_refs``.
    """
    name: str
    seed: int
    geom: Geometry
    n_max: int
    window: int
    tables: np.ndarray          # int32 [R][n_src] (n_src >= n_max; n_src > n_max: over the cap)
    refcounts: np.ndarray       # int32 [num_blocks]
    k_pool: List[np.ndarray]
    v_pool: List[np.ndarray]
    window_q: List[np.ndarray]  # [R][w][Hq][d]
    q_new: List[np.ndarray]     # [R][Hq][d]
    k_new: List[np.ndarray]     # [R][H][d]
    v_new: List[np.ndarray]     # [R][H][d]
    notes: str = ""
    extra: dict = field(default_factory=dict)
    num_blocks: Optional[np.ndarray] = None  # int32 [R] when requests hold different counts

    @property
    def num_reqs(self) -> int:
        return int(self.tables.shape[0])

    @property
    def n_src(self) -> int:
        return int(self.tables.shape[1])


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def _poison_pool(geom: Geometry) -> np.ndarray:
    shape = (geom.num_blocks, geom.num_kv_heads, geom.block_size, geom.head_dim)
    if geom.dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, BF16_NAN, dtype=np.uint16)


def make_case(name: str, seed: int, *, num_reqs: int, num_layers: int, num_kv_heads: int,
              num_q_heads: int, head_dim: int, block_size: int, n_max: int, window: int,
              num_blocks: int, dtype: str, key_scale_range: Optional[tuple] = None,
              shared_prefix_blocks: int = 0, key_kind: str = "iid", ar_rho: float = 0.9,
              planted_frac: float = 0.0, planted_scale: float = 8.0,
              n_src=None) -> CompressCase:
    """Build a seeded case.

    key_kind "iid": K ~ N(0,1) (optionally times a per (layer, head) scale
    drawn from ``key_scale_range``).  key_kind "ar1": along the logical slots
    of each (request, head, dim), k_0 = e_0, k_t = rho*k_{t-1} + sqrt(1-rho^2)*e_t,
    then a fraction ``planted_frac`` of (request, head, slot) rows, drawn
    without replacement, is multiplied by ``planted_scale``.
    ``shared_prefix_blocks`` > 0: every request's first blocks are the same
    physical ids with the same contents (refcount = num_reqs).
    ``n_src`` (default n_max): blocks each request holds, all full; more than
    n_max is a cache past the cap (e.g. a long prompt).  A list gives each
    request its own count: the table rows are then as long as the largest,
    each padded with -1, and ``num_blocks`` holds the counts.
    """
    geom = Geometry(num_layers, num_kv_heads, num_q_heads, head_dim, block_size, num_blocks, dtype)
    rng = np.random.default_rng(seed)
    R, H, Hq, d, b = num_reqs, num_kv_heads, num_q_heads, head_dim, block_size
    P = shared_prefix_blocks
    ragged = isinstance(n_src, (list, tuple, np.ndarray))
    counts = (np.asarray(n_src, dtype=np.int32) if ragged
              else np.full(R, n_max if n_src is None else int(n_src), dtype=np.int32))
    if len(counts) != R or counts.min() < n_max:
        raise ValueError("n_src must be >= n_max for every request")
    nb_req = int(counts.max())
    need = P + int(np.sum(counts - P))
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need}")
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((R, nb_req), -1, dtype=np.int32)
    tables[:, :P] = perm[:P]
    at = P
    for r in range(R):
        tables[r, P:counts[r]] = perm[at:at + counts[r] - P]
        at += counts[r] - P
    refcounts = np.zeros(num_blocks, dtype=np.int32)
    np.add.at(refcounts, tables[tables >= 0], 1)

    T = nb_req * b
    k_pool, v_pool, wq, qn, kn, vn = [], [], [], [], [], []
    for layer in range(num_layers):
        sigma = np.ones(H)
        if key_scale_range is not None:
            sigma = rng.uniform(key_scale_range[0], key_scale_range[1], size=H)
        kp = _poison_pool(geom)
        vp = _poison_pool(geom)
        shared_k = shared_v = None
        for r in range(R):
            if key_kind == "iid":
                k = rng.standard_normal((nb_req, H, b, d))
            elif key_kind == "ar1":
                eps = rng.standard_normal((H, T, d))
                k_lin = np.empty_like(eps)
                k_lin[:, 0] = eps[:, 0]
                c = np.sqrt(1.0 - ar_rho * ar_rho)
                for t in range(1, T):
                    k_lin[:, t] = ar_rho * k_lin[:, t - 1] + c * eps[:, t]
                if planted_frac > 0:
                    n_pl = int(round(planted_frac * H * T))
                    idx = rng.choice(H * T, size=n_pl, replace=False)
                    k_lin.reshape(H * T, d)[idx] *= planted_scale
                k = k_lin.reshape(H, nb_req, b, d).transpose(1, 0, 2, 3)
            else:
                raise ValueError(key_kind)
            k = k * sigma[None, :, None, None]
            v = rng.standard_normal((nb_req, H, b, d))
            if P:
                if shared_k is None:
                    shared_k, shared_v = k[:P].copy(), v[:P].copy()
                k[:P] = shared_k
                v[:P] = shared_v
            n = int(counts[r])
            kp[tables[r, :n]] = _to_storage(k[:n], dtype)
            vp[tables[r, :n]] = _to_storage(v[:n], dtype)
        k_pool.append(kp)
        v_pool.append(vp)
        wq.append(_to_storage(rng.standard_normal((R, window, Hq, d)), dtype))
        qn.append(_to_storage(rng.standard_normal((R, Hq, d)), dtype))
        kn.append(_to_storage(rng.standard_normal((R, H, d)) * sigma[None, :, None], dtype))
        vn.append(_to_storage(rng.standard_normal((R, H, d)), dtype))
    return CompressCase(name, seed, geom, n_max, window, tables, refcounts,
                        k_pool, v_pool, wq, qn, kn, vn,
                        num_blocks=counts.copy() if ragged else None)


def pool_from_logical(logical: np.ndarray, tables: np.ndarray, num_blocks: int,
                      dtype: str) -> np.ndarray:
    """Scatter logical rows [R][H][T][d] into a NaN-poisoned [nb][H][b][d] pool.

    ``tables`` [R][n] gives the physical block of each logical block; the block
    size is T / n.  Shared ids simply receive the same rows again.
    """
    R, H, T, d = logical.shape
    n = tables.shape[1]
    b = T // n
    geom = Geometry(1, H, H, d, b, num_blocks, dtype)
    pool = _poison_pool(geom)
    data = _to_storage(logical.reshape(R, H, n, b, d).transpose(0, 2, 1, 3, 4), dtype)
    for r in range(R):
        pool[tables[r]] = data[r]
    return pool


# --- the named workloads -------------------------------------------------

def case_tiny(seed: int = 101) -> CompressCase:
    """1 layer, 1 request, 2 KV / 4 query heads, d=64, fp32, b=16, N_max=8,
    w=8, pool of 16 blocks; 128 cached tokens, the pending one triggers."""
    return make_case("tiny", seed, num_reqs=1, num_layers=1, num_kv_heads=2, num_q_heads=4,
                     head_dim=64, block_size=16, n_max=8, window=8, num_blocks=16, dtype="f32")


def case_qwen3_8b_layer(seed: int = 102, num_reqs: int = 64, num_layers: int = 1) -> CompressCase:
    """Qwen3-8B-shaped layer: 8 KV / 32 query heads, d=128, bf16, b=16,
    budget 2048 (N_max=128), w=16, per-head key scale U(0.5, 2), pool 16384."""
    return make_case("qwen3_8b_budget2048", seed, num_reqs=num_reqs, num_layers=num_layers,
                     num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=16, n_max=128,
                     window=16, num_blocks=16384, dtype="bf16", key_scale_range=(0.5, 2.0))


def case_shared_prefix(seed: int = 104, num_reqs: int = 32, num_layers: int = 32,
                       num_blocks: int = 8192) -> CompressCase:
    """DeepSeek-R1-Distill-Llama-8B shape: 8 KV / 32 query heads, d=128, bf16,
    b=16, N_max=128, w=16; 32 requests share a 512-token prefix (32 blocks)."""
    return make_case("shared_prefix", seed, num_reqs=num_reqs, num_layers=num_layers,
                     num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=16, n_max=128,
                     window=16, num_blocks=num_blocks, dtype="bf16", shared_prefix_blocks=32)


def case_structured(seed: int = 105, num_reqs: int = 512, num_blocks: int = 65536) -> CompressCase:
    """Budget 4096 with AR(1) keys (rho 0.9) and 1% planted x8 keys:
    8 KV / 32 query heads, d=128, bf16, b=32, N_max=128, w=32."""
    return make_case("structured_b32", seed, num_reqs=num_reqs, num_layers=1, num_kv_heads=8,
                     num_q_heads=32, head_dim=128, block_size=32, n_max=128, window=32,
                     num_blocks=num_blocks, dtype="bf16", key_kind="ar1", ar_rho=0.9,
                     planted_frac=0.01, planted_scale=8.0)
