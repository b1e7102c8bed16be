"""GPU parity of the recorded window normalisers: zp_paged_decode_lse against
the oracle's log-sum-exp, and zp_compress_lse (scoring that reads K once,
fed with the normalisers the decode steps of the window rows record) against
the oracle's compression, to the same bar as the self-contained path.

Tolerance of the log-sum-exp: 2e-3 absolute, the decode contract's bound
(float32 dot products and sums against double).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import check_case, run_case, say
from test_gpu_parity import CASES, _case

pytestmark = pytest.mark.gpu

LSE_ATOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_paged_kv_amd as zp
    zp.lib()


def _decode_case(dtype, d, b, G, R, H, max_blocks, seed):
    return _case("lse", seed, dtype=dtype, head_dim=d, block_size=b, num_reqs=R,
                 num_kv_heads=H, num_q_heads=H * G, n_max=max_blocks, window=1,
                 num_blocks=R * max_blocks + 3)


@pytest.mark.parametrize("dtype,d,b,G,R,H", [
    ("bf16", 128, 16, 4, 10, 2),   # few units: the block list is split, merged by the combine
    ("f32", 64, 32, 2, 10, 2),
    ("bf16", 128, 16, 4, 64, 8),   # 512 workgroups: one split, merged in the decode kernel
])
def test_decode_lse_matches_oracle(dtype, d, b, G, R, H):
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    max_blocks = 12
    c = _decode_case(dtype, d, b, G, R, H, max_blocks, 220)
    rng = np.random.default_rng(221)
    seqs = rng.integers(1, max_blocks * b + 1, size=R).astype(np.int32)
    seqs[0] = 0
    seqs[-1] = max_blocks * b
    say(f"[gpu lse] decode lse {dtype} d={d} b={b} G={G} R={R} H={H}")
    dev = "cuda"
    cache = zp.KVCache([to_tensor(c.k_pool[0], dev)], [to_tensor(c.v_pool[0], dev)], H * G)
    tab = torch.from_numpy(c.tables).to(dev)
    seq_t = torch.from_numpy(seqs).to(dev)
    q = to_tensor(c.q_new[0], dev)
    ws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, max_blocks), 16),
                     dtype=torch.uint8, device=dev)
    out_plain = torch.empty((R, H * G, d), device=dev)
    out = torch.empty((R, H * G, d), device=dev)
    lse = torch.full((R, H * G), float("nan"), device=dev)
    zp.paged_decode(cache, 0, q, tab, seq_t, 1.0 / np.sqrt(d), out_plain, ws)
    zp.paged_decode(cache, 0, q, tab, seq_t, 1.0 / np.sqrt(d), out, ws, lse_out=lse)
    torch.cuda.synchronize()
    got = lse.cpu().numpy()
    want = oracle.decode_lse(c.k_pool[0], c.q_new[0], c.tables, seqs, num_q_heads=H * G)
    assert np.all(np.isneginf(got[0])), "empty request must give -inf"
    err = np.abs(got[1:] - want[1:])
    assert np.isfinite(got[1:]).all() and err.max() <= LSE_ATOL, err.max()
    # the attention output is the same computation with or without the lse
    assert torch.equal(out, out_plain)


def test_decode_lse_row_map_skips_and_scatters():
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    R, H, G, d, b, max_blocks = 6, 2, 2, 64, 16, 5
    c = _decode_case("bf16", d, b, G, R, H, max_blocks, 222)
    seqs = np.array([80, 1, 17, 33, 64, 79], dtype=np.int32)
    rows = np.array([7, -1, 0, 9, 3, 12], dtype=np.int32)   # 12 is past the 10-row buffer
    say("[gpu lse] decode lse row map")
    dev = "cuda"
    cache = zp.KVCache([to_tensor(c.k_pool[0], dev)], [to_tensor(c.v_pool[0], dev)], H * G)
    ws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, max_blocks), 16),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((R, H * G, d), device=dev)
    lse = torch.full((10, H * G), float("nan"), device=dev)
    q = to_tensor(c.q_new[0], dev)
    q_rec = torch.full((10, H * G, d), float("nan"), dtype=q.dtype, device=dev)
    zp.paged_decode(cache, 0, q, torch.from_numpy(c.tables).to(dev),
                    torch.from_numpy(seqs).to(dev), 1.0 / np.sqrt(d), out, ws, lse_out=lse,
                    lse_rows=torch.from_numpy(rows).to(dev), q_out=q_rec)
    torch.cuda.synchronize()
    got = lse.cpu().numpy()
    # the query is recorded bit for bit in the same rows (the query slots)
    for rw in range(10):
        src = [r for r, x in enumerate(rows) if x == rw]
        if src:
            assert torch.equal(q_rec[rw].view(torch.int16), q[src[0]].view(torch.int16))
        else:
            assert torch.isnan(q_rec[rw].float()).all()
    want = oracle.decode_lse(c.k_pool[0], c.q_new[0], c.tables, seqs, num_q_heads=H * G)
    written = {int(rw): r for r, rw in enumerate(rows) if 0 <= rw < 10}
    for rw in range(10):
        if rw in written:
            assert np.abs(got[rw] - want[written[rw]]).max() <= LSE_ATOL
        else:
            assert np.isnan(got[rw]).all(), f"row {rw} must stay untouched"


@pytest.mark.parametrize("name", list(CASES))
def test_compress_with_recorded_lse_matches_oracle(name):
    case = CASES[name]()
    g = case.geom
    say(f"[gpu lse] compress with recorded normalisers: {name} R={case.num_reqs} "
        f"L={g.num_layers} H={g.num_kv_heads} Hq={g.num_q_heads} d={g.head_dim} "
        f"b={g.block_size} n_max={case.n_max} w={case.window} {g.dtype}")
    run = run_case(case, recorded_lse=True)
    stats = check_case(case, run)
    say(f"[gpu lse] {name}: ok {stats}")


def test_qwen3_8b_layer_full_size_recorded_lse():
    case = synth.case_qwen3_8b_layer()
    say("[gpu lse] qwen3-8b layer, 64 requests, budget 2048, recorded normalisers")
    run = run_case(case, recorded_lse=True)
    stats = check_case(case, run)
    say(f"[gpu lse] qwen3-8b layer: ok {stats}")
