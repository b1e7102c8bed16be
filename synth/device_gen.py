"""Seeded synthetic workloads generated directly in device memory.

The full-size workloads (tens of GB of K/V) are too large to draw on the host
with NumPy, so their random rows come from torch's device generator, seeded.
The recipes are the host ones (``synth.make_case``): block ids from a seeded
permutation of the pool, K ~ N(0,1) times a per (layer, head) scale, or AR(1)
keys along each request's logical slots with planted large rows, V and the
queries ~ N(0,1), everything rounded to the cache dtype (RNE), unreferenced
blocks poisoned with NaN.  The draws differ from the host generator's (another
stream of random numbers), not the distribution.

Nothing here computes any part of the method.  The oracle reads these bytes
back to the host (``synth.device.to_numpy``) for the sampled checks.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import Geometry


@dataclass
class DeviceCase:
    name: str
    seed: int
    geom: Geometry
    n_max: int
    window: int
    tables: np.ndarray        # int32 [R][n_src] physical block ids (host), n_src >= n_max
    refcounts: np.ndarray     # int32 [num_blocks] (host)
    seq_lens: np.ndarray      # int32 [R] cached tokens before the pending one
    k_pool: List[torch.Tensor] = field(default_factory=list)  # per layer [nb][H][b][d]
    v_pool: List[torch.Tensor] = field(default_factory=list)
    window_q: List[torch.Tensor] = field(default_factory=list)  # per layer [R][w][Hq][d]
    q_new: List[torch.Tensor] = field(default_factory=list)     # per layer [R][Hq][d]
    k_new: List[torch.Tensor] = field(default_factory=list)     # per layer [R][H][d]
    v_new: List[torch.Tensor] = field(default_factory=list)
    notes: str = ""

    @property
    def num_reqs(self) -> int:
        return int(self.tables.shape[0])

    @property
    def n_src(self) -> int:
        return int(self.tables.shape[1])


def _tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _ar1_rows(gen, shape, rho: float, device) -> torch.Tensor:
    """[..., T, d] rows with x_0 = e_0 and x_t = rho*x_{t-1} + sqrt(1-rho^2)*e_t
    along T, by a log-depth doubling scan (float32)."""
    e = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    c = float(np.sqrt(1.0 - rho * rho))
    x = e
    x[..., 1:, :] *= c
    T = shape[-2]
    s, a = 1, rho
    while s < T:
        y = x.clone()
        y[..., s:, :] += a * x[..., :-s, :]
        x = y
        s *= 2
        a = a * a
    return x


def make_device_case(name: str, seed: int, device, *, num_reqs: int, num_layers: int,
                     num_kv_heads: int, num_q_heads: int, head_dim: int, block_size: int,
                     n_max: int, window: int, num_blocks: int, dtype: str = "bf16",
                     key_scale_range: Optional[tuple] = (0.5, 2.0), shared_prefix_blocks: int = 0,
                     key_kind: str = "iid", ar_rho: float = 0.9, planted_frac: float = 0.0,
                     planted_scale: float = 8.0, seq_lens: Optional[np.ndarray] = None,
                     chunk_reqs: int = 32, n_src: Optional[int] = None) -> DeviceCase:
    """Every request holds n_src (default n_max) blocks, the first
    ``shared_prefix_blocks`` of them shared by all requests; ``seq_lens``
    (default n_src * block_size) says how many of its slots are cached."""
    geom = Geometry(num_layers, num_kv_heads, num_q_heads, head_dim, block_size, num_blocks, dtype)
    R, H, Hq, d, b = num_reqs, num_kv_heads, num_q_heads, head_dim, block_size
    P = shared_prefix_blocks
    nb_req = n_max if n_src is None else int(n_src)
    if nb_req < n_max:
        raise ValueError("n_src must be >= n_max")
    need = P + R * (nb_req - P)
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {need}")
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.empty((R, nb_req), dtype=np.int32)
    tables[:, :P] = perm[:P]
    tables[:, P:] = perm[P:need].reshape(R, nb_req - P)
    refcounts = np.zeros(num_blocks, dtype=np.int32)
    np.add.at(refcounts, tables.reshape(-1), 1)
    if seq_lens is None:
        seq_lens = np.full(R, nb_req * b, dtype=np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = _tdtype(dtype)
    used = torch.zeros(num_blocks, dtype=torch.bool, device=device)
    used[torch.from_numpy(tables.reshape(-1).astype(np.int64)).to(device)] = True
    unused = ~used
    T = nb_req * b
    case = DeviceCase(name, seed, geom, n_max, window, tables, refcounts, seq_lens)
    for _ in range(num_layers):
        sigma = torch.ones(H, device=device)
        if key_scale_range is not None:
            lo, hi = key_scale_range
            sigma = lo + (hi - lo) * torch.rand(H, generator=gen, device=device)
        kp = torch.empty((num_blocks, H, b, d), dtype=tdt, device=device)
        vp = torch.empty((num_blocks, H, b, d), dtype=tdt, device=device)
        if key_kind == "iid":
            for c0 in range(0, num_blocks, 4096):
                c1 = min(num_blocks, c0 + 4096)
                k = torch.randn((c1 - c0, H, b, d), generator=gen, device=device)
                kp[c0:c1] = (k * sigma[None, :, None, None]).to(tdt)
        elif key_kind == "ar1":
            if P:
                raise ValueError("AR(1) keys with a shared prefix are not a workload here")
            kp.fill_(float("nan"))
            for r0 in range(0, R, chunk_reqs):
                r1 = min(R, r0 + chunk_reqs)
                x = _ar1_rows(gen, (r1 - r0, H, T, d), ar_rho, device)
                if planted_frac > 0:
                    n_pl = int(round(planted_frac * H * T))
                    flat = x.view(r1 - r0, H * T, d)
                    for i in range(r1 - r0):
                        idx = torch.randperm(H * T, generator=gen, device=device)[:n_pl]
                        flat[i, idx] *= planted_scale
                x = x * sigma[None, :, None, None]
                blocks = x.view(r1 - r0, H, nb_req, b, d).permute(0, 2, 1, 3, 4).to(tdt)
                ids = torch.from_numpy(tables[r0:r1].astype(np.int64)).to(device)
                kp.index_copy_(0, ids.reshape(-1), blocks.reshape(-1, H, b, d))
                del x, blocks
        else:
            raise ValueError(key_kind)
        for c0 in range(0, num_blocks, 4096):
            c1 = min(num_blocks, c0 + 4096)
            vp[c0:c1] = torch.randn((c1 - c0, H, b, d), generator=gen, device=device).to(tdt)
        kp[unused] = float("nan")
        vp[unused] = float("nan")
        case.k_pool.append(kp)
        case.v_pool.append(vp)
        case.window_q.append(torch.randn((R, window, Hq, d), generator=gen, device=device).to(tdt))
        case.q_new.append(torch.randn((R, Hq, d), generator=gen, device=device).to(tdt))
        case.k_new.append((torch.randn((R, H, d), generator=gen, device=device)
                           * sigma[None, :, None]).to(tdt))
        case.v_new.append(torch.randn((R, H, d), generator=gen, device=device).to(tdt))
    return case


# --- the full-size workloads --------------------------------------------

def case_qwen3_8b_layer_batches(device, n: int, seed: int = 102, num_reqs: int = 64) -> DeviceCase:
    """n independent batches of the Qwen3-8B-shaped layer at budget 2048 (64
    requests at N_max = 128, b = 16, w = 16, 8 KV / 32 query heads, d = 128,
    bf16, per-head key scale U(0.5, 2), pool 16384), as the n "layers" of one
    case: one seeded set of block tables, each batch its own pools, window
    queries, pending token and decode query."""
    return make_device_case("qwen3_8b_budget2048", seed, device, num_reqs=num_reqs, num_layers=n,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=16, n_max=128,
                            window=16, num_blocks=16384)


def case_mix_device(device, seed: int = 103, num_reqs: int = 256, num_layers: int = 36,
                    compress_frac: float = 0.1) -> DeviceCase:
    """Continuous-batching mix on the Qwen3-8B shape: 256 requests x 36 layers,
    pool 256 * N_max blocks; a seeded 10% of the requests hold 2048 cached
    tokens (they compress), the others hold U[64, 2047]."""
    rng = np.random.default_rng(seed + 7)
    n_c = int(round(compress_frac * num_reqs))
    comp = np.sort(rng.choice(num_reqs, size=n_c, replace=False))
    lens = rng.integers(64, 2048, size=num_reqs).astype(np.int32)
    lens[comp] = 2048
    case = make_device_case("mix_qwen3_8b", seed, device, num_reqs=num_reqs, num_layers=num_layers,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=16, n_max=128,
                            window=16, num_blocks=num_reqs * 128, seq_lens=lens)
    case.notes = f"compressing requests: {comp.tolist()}"
    return case


def case_shared_prefix_device(device, seed: int = 104, num_reqs: int = 32,
                              num_layers: int = 32) -> DeviceCase:
    """32 requests x 32 layers sharing a 32-block (512-token) prefix, 96
    private blocks each, all at 2048 cached; pool 8192."""
    return make_device_case("shared_prefix", seed, device, num_reqs=num_reqs, num_layers=num_layers,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=16, n_max=128,
                            window=16, num_blocks=8192, key_scale_range=None,
                            shared_prefix_blocks=32)


def case_over_cap_device(device, seed: int = 106, num_reqs: int = 64,
                         n_src: int = 160) -> DeviceCase:
    """Qwen3-8B shape past the cap: 64 requests each holding a 2560-token
    prompt (160 full blocks) compressed to budget 2048 (N_max = 128, w = 16);
    per-head key scale U(0.5, 2); pool 16384."""
    return make_device_case("over_cap_qwen3_8b", seed, device, num_reqs=num_reqs, num_layers=1,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=16, n_max=128,
                            window=16, num_blocks=16384, n_src=n_src)


def case_structured_device(device, seed: int = 105, num_reqs: int = 512) -> DeviceCase:
    """512 requests, budget 4096 (b = 32, N_max = 128, w = 32), AR(1) keys
    (rho 0.9) with 1% of rows scaled x8; pool 65536."""
    return make_device_case("structured_b32", seed, device, num_reqs=num_reqs, num_layers=1,
                            num_kv_heads=8, num_q_heads=32, head_dim=128, block_size=32, n_max=128,
                            window=32, num_blocks=65536, key_scale_range=None, key_kind="ar1",
                            ar_rho=0.9, planted_frac=0.01, planted_scale=8.0)
