"""GPU parity of the all-pairs redundancy (zp_redundancy_all, the pairwise
score the Lightning Redundancy Score replaces) against the oracle: within
1e-3 absolute, the redundancy bar of the compression parity (it is a mean
of cosines, bounded and crossing zero)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import R_ATOL, say
from synth.device import to_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_paged_kv_amd as zp
    zp.lib()


@pytest.mark.parametrize("dtype,d,b,n_blocks,key_kind", [
    ("bf16", 128, 16, 37, "iid"),     # T = 592: partial last chunk of 128 keys
    ("f32", 64, 32, 9, "iid"),
    ("bf16", 64, 16, 64, "ar1"),      # correlated keys: large positive scores
    ("f32", 128, 16, 3, "iid"),       # T = 48: fewer row tiles than waves
    ("bf16", 128, 32, 128, "ar1"),    # T = 4096, the structured budget-4096 length
])
def test_redundancy_all_matches_oracle(dtype, d, b, n_blocks, key_kind):
    import compressed_paged_kv_amd as zp
    c = synth.make_case("rall", 230 + n_blocks, num_reqs=2, num_layers=1, num_kv_heads=2,
                        num_q_heads=2, head_dim=d, block_size=b, n_max=n_blocks, window=1,
                        num_blocks=2 * n_blocks + 5, dtype=dtype, key_kind=key_kind,
                        planted_frac=0.01 if key_kind == "ar1" else 0.0)
    T = n_blocks * b
    say(f"[gpu redundancy] all pairs {dtype} d={d} b={b} T={T} {key_kind}")
    dev = "cuda"
    kp = to_tensor(c.k_pool[0], dev)
    cache = zp.KVCache([kp], [to_tensor(c.v_pool[0], dev)], 2)
    out = torch.full((2, 2, T), float("nan"), device=dev)
    zp.redundancy_all(cache, 0, torch.from_numpy(c.tables).to(dev), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.redundancy_all(c.k_pool[0], c.tables)
    err = np.abs(got - want)
    assert np.isfinite(got).all() and err.max() <= R_ATOL, err.max()
    say(f"[gpu redundancy] max abs error {err.max():.2e}")


def test_redundancy_all_qwen3_layer_sampled():
    """The Qwen3-8B-shaped layer (64 requests, T = 2048): all heads of four
    sampled requests against the oracle."""
    import compressed_paged_kv_amd as zp
    case = synth.case_qwen3_8b_layer()
    say("[gpu redundancy] qwen3-8b layer, 64 requests, T = 2048")
    dev = "cuda"
    cache = zp.KVCache([to_tensor(case.k_pool[0], dev)], [to_tensor(case.v_pool[0], dev)], 32)
    out = torch.empty((64, 8, 2048), device=dev)
    zp.redundancy_all(cache, 0, torch.from_numpy(case.tables).to(dev), out)
    torch.cuda.synchronize()
    rs = [0, 17, 42, 63]
    want = oracle.redundancy_all(case.k_pool[0], case.tables[rs])
    err = np.abs(out.cpu().numpy()[rs] - want)
    assert err.max() <= R_ATOL, err.max()


@pytest.mark.parametrize("dtype,d,b", [("bf16", 128, 16), ("f32", 64, 32)])
def test_redundancy_all_with_zero_norm_keys(dtype, d, b):
    """Zero keys (cosine 0 with everything, redundancy 0 themselves): a few
    rows of one block and one whole block of request 0, one row of head 1 of
    request 1; the other keys' means still divide by T - 1."""
    import compressed_paged_kv_amd as zp
    n_blocks = 24
    c = synth.make_case("rall0", 260, num_reqs=2, num_layers=1, num_kv_heads=2, num_q_heads=2,
                        head_dim=d, block_size=b, n_max=n_blocks, window=1,
                        num_blocks=2 * n_blocks + 5, dtype=dtype)
    zero = np.float32(0) if dtype == "f32" else np.uint16(0)
    for h in range(2):
        c.k_pool[0][c.tables[0, 3], h, [0, 2, b - 1], :] = zero
        c.k_pool[0][c.tables[0, 7], h] = zero
    c.k_pool[0][c.tables[1, 0], 1, 0, :] = zero
    T = n_blocks * b
    say(f"[gpu redundancy] zero-norm keys {dtype} d={d} b={b} T={T}")
    dev = "cuda"
    cache = zp.KVCache([to_tensor(c.k_pool[0], dev)], [to_tensor(c.v_pool[0], dev)], 2)
    out = torch.full((2, 2, T), float("nan"), device=dev)
    zp.redundancy_all(cache, 0, torch.from_numpy(c.tables).to(dev), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.redundancy_all(c.k_pool[0], c.tables)
    np.testing.assert_array_equal(got[0, :, 7 * b:8 * b], 0.0)
    np.testing.assert_array_equal(got[0, :, 3 * b + np.array([0, 2, b - 1])], 0.0)
    assert got[1, 1, 0] == 0.0
    err = np.abs(got - want)
    assert np.isfinite(got).all() and err.max() <= R_ATOL, err.max()
