"""The synthetic inputs follow their stated recipe (CPU).

Block ids a seeded permutation of the pool, unreferenced blocks NaN, a shared
prefix the same ids and bytes in every request, rows of requests holding
different block counts padded with -1; per (layer, head) key scales within
the stated range; AR(1) keys with the stated lag-1 correlation and unit
variance, and the stated fraction of planted rows at the stated scale; the
device generator's log-depth AR(1) scan equal to the sequential recurrence.
"""
import numpy as np
import torch

import synth
from synth.device_gen import _ar1_rows


def _logical(pool, tables, r, n):
    """[H][n*b][d] float32 rows of request r's first n blocks."""
    x = synth.bf16_bits_to_f32(pool) if pool.dtype == np.uint16 else pool
    blk = x[tables[r, :n]]                      # [n][H][b][d]
    return blk.transpose(1, 0, 2, 3).reshape(blk.shape[1], -1, blk.shape[3])


def test_tables_pool_and_shared_prefix():
    c = synth.make_case("rc", 11, num_reqs=4, num_layers=2, num_kv_heads=2, num_q_heads=4,
                        head_dim=64, block_size=16, n_max=6, window=8, num_blocks=40, dtype="bf16",
                        shared_prefix_blocks=2)
    ids = c.tables.reshape(-1)
    assert ids.min() >= 0 and ids.max() < 40
    assert np.all(c.tables[:, :2] == c.tables[0, :2])                 # the prefix ids
    assert len(set(c.tables[:, 2:].reshape(-1).tolist())) == 4 * 4    # private ids all distinct
    assert np.all(c.refcounts[c.tables[0, :2]] == 4) and c.refcounts.sum() == 4 * 6
    unused = np.setdiff1d(np.arange(40), ids)
    for pool in c.k_pool + c.v_pool:
        assert np.isnan(synth.bf16_bits_to_f32(pool[unused])).all()
        assert np.isfinite(synth.bf16_bits_to_f32(pool[ids])).all()
    for l in range(2):      # the prefix holds the same rows for every request
        k0 = _logical(c.k_pool[l], c.tables, 0, 2)
        for r in range(1, 4):
            np.testing.assert_array_equal(_logical(c.k_pool[l], c.tables, r, 2), k0)


def test_rows_of_different_block_counts_are_padded():
    c = synth.make_case("rp", 12, num_reqs=3, num_layers=1, num_kv_heads=1, num_q_heads=2,
                        head_dim=64, block_size=16, n_max=4, window=4, num_blocks=40,
                        dtype="f32", n_src=[4, 9, 6])
    assert c.tables.shape == (3, 9) and c.num_blocks.tolist() == [4, 9, 6]
    for r, n in enumerate([4, 9, 6]):
        assert np.all(c.tables[r, :n] >= 0) and np.all(c.tables[r, n:] == -1)


def test_per_head_key_scales_within_the_range():
    c = synth.make_case("ks", 13, num_reqs=8, num_layers=3, num_kv_heads=4, num_q_heads=8,
                        head_dim=128, block_size=16, n_max=16, window=16, num_blocks=140,
                        dtype="f32", key_scale_range=(0.5, 2.0))
    sds = []
    for l in range(3):
        k = np.stack([_logical(c.k_pool[l], c.tables, r, 16) for r in range(8)])   # [R][H][T][d]
        v = np.stack([_logical(c.v_pool[l], c.tables, r, 16) for r in range(8)])
        sd = k.transpose(1, 0, 2, 3).reshape(4, -1).std(axis=1)
        assert np.all(sd > 0.5 * 0.97) and np.all(sd < 2.0 * 1.03)
        assert abs(v.std() - 1.0) < 0.02 and abs(k.mean()) < 0.02
        sds.extend(sd.tolist())
    assert max(sds) / min(sds) > 1.5          # the scales differ: a dropped scale fails here


def test_ar1_keys_and_planted_rows():
    """rho = 0.9 along each request's logical slots (lag-1 correlation of the
    unplanted rows), unit variance, and 1 % of the rows times 8."""
    T, d = 1024, 64
    c = synth.make_case("ar", 14, num_reqs=4, num_layers=1, num_kv_heads=2, num_q_heads=4,
                        head_dim=d, block_size=32, n_max=T // 32, window=32, num_blocks=140,
                        dtype="f32", key_kind="ar1", ar_rho=0.9, planted_frac=0.01,
                        planted_scale=8.0)
    k = np.stack([_logical(c.k_pool[0], c.tables, r, T // 32) for r in range(4)])   # [R][H][T][d]
    norms = np.linalg.norm(k, axis=-1)
    planted = norms > 4.0 * np.sqrt(d)        # a planted row is 8x a row of norm ~ sqrt(d)
    frac = planted.mean()
    assert abs(frac - 0.01) < 0.003, frac
    ok = ~planted
    pair = ok[..., 1:] & ok[..., :-1]
    x0, x1 = k[..., :-1, :][pair], k[..., 1:, :][pair]
    rho = float((x0 * x1).sum() / np.sqrt((x0 * x0).sum() * (x1 * x1).sum()))
    assert abs(rho - 0.9) < 0.01, rho
    assert abs(k[ok].var() - 1.0) < 0.05


def test_device_ar1_scan_is_the_recurrence():
    """The log-depth doubling scan gives x_0 = e_0, x_t = rho x_{t-1} +
    sqrt(1 - rho^2) e_t on the same draws (torch's generator replayed)."""
    rho, shape = 0.9, (3, 300, 8)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(5)
    state = gen.get_state()
    x = _ar1_rows(gen, shape, rho, "cpu").numpy().astype(np.float64)
    gen.set_state(state)
    e = torch.randn(shape, generator=gen, device="cpu", dtype=torch.float32).numpy().astype(np.float64)
    want = np.empty_like(e)
    want[:, 0] = e[:, 0]
    c = np.sqrt(1.0 - rho * rho)
    for t in range(1, shape[1]):
        want[:, t] = rho * want[:, t - 1] + c * e[:, t]
    np.testing.assert_allclose(x, want, rtol=0, atol=2e-5)
