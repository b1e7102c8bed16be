"""GPU parity: the HIP path against the CPU oracle, element by element.

Every case prints its name and shape before it touches the GPU.  Shapes
span several score chunks and compaction tiles with ragged tails (n_max not a
multiple of the 512-token chunk, G*w not a multiple of 16, C not a multiple
of 256), both block sizes, both head dims, both element types and group
sizes 1..8; the Qwen3-8B-shaped layer runs at its full size (64 requests,
budget 2048) in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import DECODE_ATOL, check_case, run_case, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_paged_kv_amd as zp
    zp.lib()  # raises if the HIP library is missing


def _case(name, seed, **kw):
    base = dict(num_reqs=2, num_layers=1, num_kv_heads=2, num_q_heads=4, head_dim=128,
                block_size=16, n_max=12, window=16, num_blocks=64, dtype="bf16")
    base.update(kw)
    return synth.make_case(name, seed, **base)


CASES = {
    # the tiny CPU-checkable workload: fp32, d=64, b=16, N_max=8, w=8, G=2
    "tiny": lambda: synth.case_tiny(),
    # ragged: 37 blocks -> two score chunks, the second partial; G*w = 64
    "bf16_d128_b16_ragged": lambda: _case("r1", 201, num_reqs=3, n_max=37, num_blocks=160,
                                          num_kv_heads=2, num_q_heads=8),
    # b=32, w=32, G=4 -> 128 window rows (8 row tiles), d=64
    "bf16_d64_b32_rows128": lambda: _case("r2", 202, head_dim=64, block_size=32, n_max=20,
                                          window=32, num_q_heads=8, num_blocks=64),
    # fp32, b=32, w=5, G=1 -> 5 rows padded to one tile, d=128
    "f32_d128_b32_w5": lambda: _case("r3", 203, dtype="f32", block_size=32, n_max=9, window=5,
                                     num_q_heads=2, num_blocks=40),
    # G=8 (decode splits the group over two workgroups), 128 rows
    "bf16_g8": lambda: _case("r4", 204, num_kv_heads=1, num_q_heads=8, n_max=16, num_blocks=40),
    # f32, d=64, b=16, w=1 (a single window query), G=4
    "f32_d64_w1": lambda: _case("r5", 205, dtype="f32", head_dim=64, window=1, n_max=10,
                                num_q_heads=8, num_blocks=40),
    # two layers, shared prefix of 3 blocks among 4 requests (new target blocks)
    "shared_prefix_2layers": lambda: _case("r6", 206, num_reqs=4, num_layers=2, n_max=12,
                                           num_blocks=80, shared_prefix_blocks=3),
    # per-head key scales as in the Qwen3-8B-shaped workload, longer cache
    "bf16_scaled_keys": lambda: _case("r7", 207, num_reqs=2, n_max=64, num_kv_heads=2,
                                      num_q_heads=8, num_blocks=160, key_scale_range=(0.5, 2.0)),
    # AR(1) keys with planted x8 keys (structured budget-4096 shape, reduced)
    "ar1_planted_b32": lambda: _case("r8", 208, block_size=32, window=32, n_max=24,
                                     num_q_heads=8, num_blocks=64, key_kind="ar1",
                                     planted_frac=0.01),
    # long caches: more than 64 blocks per wave in the scoring kernel, one row
    # group (G*w = 64, 300 blocks) and two row groups (G*w = 128, 200 blocks)
    "bf16_long_300_blocks": lambda: _case("r9", 212, num_reqs=1, num_kv_heads=1, num_q_heads=4,
                                          n_max=300, num_blocks=310),
    "bf16_long_200_blocks_rows128": lambda: _case("r10", 213, num_reqs=1, num_kv_heads=1,
                                                  num_q_heads=8, n_max=200, num_blocks=210),
    # caches past the cap (n_src > n_max): E = (n_src - n_max + 1) b evictions per
    # head (above the small-E sizes), surplus blocks released; one with a
    # shared prefix and two layers, one at b=32 with two row groups
    "over_cap_bf16_3_extra": lambda: _case("o1", 214, num_reqs=3, n_max=12, n_src=15,
                                           num_blocks=64),
    "over_cap_prefix_2layers": lambda: _case("o2", 215, num_reqs=3, num_layers=2, n_max=10,
                                             n_src=16, num_blocks=80, shared_prefix_blocks=2),
    "over_cap_b32_rows128": lambda: _case("o3", 216, head_dim=64, block_size=32, window=32,
                                          num_q_heads=8, n_max=8, n_src=20, num_blocks=48),
    "over_cap_f32_d64_many": lambda: _case("o4", 217, dtype="f32", head_dim=64, n_max=6,
                                           n_src=60, num_blocks=130),
    # the limits the host accepts: 8192 cached slots (512 blocks of 16) with one
    # row group, 4096 slots with 128 window rows (two row groups), and 1024
    # evictions per head (a cache 63 blocks past the cap)
    "max_slots_8192": lambda: _case("m1", 218, num_reqs=1, num_kv_heads=1, num_q_heads=4,
                                    n_max=512, num_blocks=520),
    "max_slots_4096_rows128": lambda: _case("m2", 219, num_reqs=1, num_kv_heads=1,
                                            num_q_heads=8, n_max=256, num_blocks=260),
    "max_evictions_1024": lambda: _case("m3", 220, num_reqs=2, head_dim=64, n_max=20, n_src=83,
                                        num_blocks=180),
    # more (layer, request, head) units than two per compute unit (576 on a
    # 256-CU MI355X): the fused compaction streams K instead of loading it
    # normally
    "units_576_streamed_k": lambda: _case("m6", 226, num_reqs=24, num_layers=3, num_kv_heads=8,
                                          num_q_heads=16, head_dim=64, n_max=6, num_blocks=200),
    # more layers than one launch carries (48): the compression runs in two
    # launches over layer chunks
    "layers_50_two_launches": lambda: _case("m7", 228, num_reqs=2, num_layers=50, num_kv_heads=1,
                                            num_q_heads=2, head_dim=64, n_max=4, window=4,
                                            num_blocks=12),
    # one call over requests holding different block counts (rows padded
    # with -1): at the cap and past it side by side, with a shared prefix and
    # two layers; b=32 with two row groups; fp32 from 6 to 60 blocks; and
    # 1024 evictions next to a request at the cap
    "mixed_counts_prefix_2layers": lambda: _case("x1", 230, num_reqs=4, num_layers=2, n_max=10,
                                                 n_src=[10, 13, 11, 16], num_blocks=90,
                                                 shared_prefix_blocks=2),
    "mixed_counts_b32_rows128": lambda: _case("x2", 231, head_dim=64, block_size=32, window=32,
                                              num_reqs=3, num_q_heads=8, n_max=8,
                                              n_src=[8, 20, 9], num_blocks=64),
    "mixed_counts_f32_d64": lambda: _case("x3", 232, dtype="f32", head_dim=64, num_reqs=3,
                                          n_max=6, n_src=[60, 6, 30], num_blocks=120),
    "mixed_counts_max_evictions": lambda: _case("x4", 233, head_dim=64, n_max=20, n_src=[83, 20],
                                                num_blocks=140),
    # 16 keys per selecting thread: 4096 slots exactly, and a ragged 3200
    "slots_4096_rows64": lambda: _case("m4", 224, num_reqs=2, num_kv_heads=1, num_q_heads=4,
                                       n_max=256, num_blocks=520),
    "slots_3200_rows32_f32": lambda: _case("m5", 225, dtype="f32", head_dim=64, num_reqs=1,
                                           num_kv_heads=2, num_q_heads=4, n_max=200,
                                           num_blocks=210),
}


@pytest.mark.parametrize("name", list(CASES))
def test_compress_and_decode_match_oracle(name):
    case = CASES[name]()
    g = case.geom
    say(f"[gpu parity] {name}: R={case.num_reqs} L={g.num_layers} H={g.num_kv_heads} "
        f"Hq={g.num_q_heads} d={g.head_dim} b={g.block_size} n_max={case.n_max} "
        f"w={case.window} dtype={g.dtype}")
    run = run_case(case)
    stats = check_case(case, run)
    say(f"[gpu parity] {name}: ok {stats}")


def _exact_tie_case(dtype, d, b, n_max, w):
    """Zero window queries and, inside every block, keys along distinct
    coordinate axes: every logit is 0 and every in-block cosine is exactly 0,
    so all candidates carry the same score and the tie rule alone decides."""
    c = _case("tie", 209, dtype=dtype, head_dim=d, block_size=b, n_max=n_max, window=w,
              num_blocks=4 * n_max)
    R, H = c.num_reqs, c.geom.num_kv_heads
    T = n_max * b
    K = np.zeros((R, H, T, d))
    for j in range(T):
        K[:, :, j, j % b] = 1.0 + (j % 3)
    c.k_pool[0] = synth.pool_from_logical(K, c.tables, c.geom.num_blocks, dtype)
    c.window_q[0] = np.zeros_like(c.window_q[0])
    return c


@pytest.mark.parametrize("dtype,d,b,n_max,w", [("bf16", 128, 16, 20, 16), ("f32", 64, 16, 8, 8),
                                               ("bf16", 64, 32, 9, 7), ("f32", 64, 16, 4, 8)])
def test_exact_ties_keep_the_lower_slots(dtype, d, b, n_max, w):
    case = _exact_tie_case(dtype, d, b, n_max, w)
    say(f"[gpu parity] exact tie {dtype} d={d} b={b} n_max={n_max} w={w}")
    run = run_case(case)
    T, k_keep = n_max * b, (n_max - 1) * b
    C = T - w
    E = C - (k_keep - w)
    want = np.array(list(range(C - E)) + list(range(C, T)))
    assert np.all(run.R[0] == 0.0)
    cand = run.s[0][..., :C]
    assert np.all(cand == cand[..., :1])          # bit-identical scores
    for r in range(case.num_reqs):
        for h in range(case.geom.num_kv_heads):
            np.testing.assert_array_equal(run.kept[0, r, h], want)
    check_case(case, run)


def test_ties_at_the_threshold_below_some_lower_scores():
    """The exact-tie cache with, in the second block of every head, keys
    0..7 made equal: their cosines are 1, so they score below every other
    candidate and go first, and the remaining E - 8 evictions fall among
    the equal scores -- the highest slots of those."""
    case = _exact_tie_case("bf16", 128, 16, 20, 16)
    say("[gpu parity] 8 lower scores, then exact ties at the threshold")
    g = case.geom
    b, d = g.block_size, g.head_dim
    for r in range(case.num_reqs):
        blk = int(case.tables[r, 1])
        for h in range(g.num_kv_heads):
            row = np.zeros(d, dtype=np.float32)
            row[0] = 1.0
            case.k_pool[0][blk, h, :8] = synth.f32_to_bf16_bits(np.tile(row, (8, 1)))
    run = run_case(case)
    n_max, w = case.n_max, case.window
    T, k_keep = n_max * b, (n_max - 1) * b
    C = T - w
    E = C - (k_keep - w)
    gone = set(range(b, b + 8)) | set(range(C - (E - 8), C))
    want = np.array([j for j in range(T) if j not in gone])
    assert len(want) == k_keep
    for r in range(case.num_reqs):
        for h in range(g.num_kv_heads):
            np.testing.assert_array_equal(run.kept[0, r, h], want)
    check_case(case, run)


def _zero_key_case(dtype, d, b):
    """Keys of zero norm (cosine 0 with every other key, so they add nothing
    to their neighbours' redundancy and have redundancy 0 themselves): in
    request 0 three rows of its third block (every head) and the whole of
    its fifth block; in request 1 the first row of head 1 only, and the row
    just before the window."""
    c = _case("zero", 227, dtype=dtype, head_dim=d, block_size=b, n_max=12, window=16,
              num_q_heads=8, num_blocks=64)
    zero = np.float32(0) if dtype == "f32" else np.uint16(0)
    T, w = c.n_max * b, c.window
    rows = {0: [(2, h, o) for h in range(2) for o in (1, 5, 6)] + [(4, h, o) for h in range(2)
                                                                  for o in range(b)],
            1: [(0, 1, 0), ((T - w - 1) // b, 0, (T - w - 1) % b)]}
    for r, lst in rows.items():
        for n, h, o in lst:
            c.k_pool[0][c.tables[r, n], h, o, :] = zero
    return c, rows


@pytest.mark.parametrize("dtype,d,b", [("bf16", 128, 16), ("f32", 64, 32), ("bf16", 64, 32)])
def test_zero_norm_keys_have_zero_cosines(dtype, d, b):
    case, rows = _zero_key_case(dtype, d, b)
    say(f"[gpu parity] zero-norm keys {dtype} d={d} b={b}")
    run = run_case(case)
    for r, lst in rows.items():
        for n, h, o in lst:
            assert run.R[0, r, h, n * b + o] == 0.0, (r, h, n, o)
    # the all-zero block: every cosine in it is 0
    np.testing.assert_array_equal(run.R[0, 0, :, 4 * b:5 * b], 0.0)
    check_case(case, run)


def _max_shift_case():
    """Window queries along one direction u per head and the keys of every
    request's first block along -2u: those 16 slots get by far the smallest
    importance, so the whole first block is evicted and every survivor moves
    up by b slots -- the largest in-place shift, where each compaction tile
    reads the rows the tile after it overwrites."""
    c = _case("shift", 223, num_reqs=2, n_max=20, num_kv_heads=2, num_q_heads=8, num_blocks=64)
    g = c.geom
    H, Hq, d, b = g.num_kv_heads, g.num_q_heads, g.head_dim, g.block_size
    G = Hq // H
    rng = np.random.default_rng(2230)
    u = rng.standard_normal((H, d))
    wq = np.repeat(u, G, axis=0)[None, None] + 0.3 * rng.standard_normal((c.num_reqs, c.window, Hq, d))
    c.window_q[0] = synth.f32_to_bf16_bits(wq.astype(np.float32))
    for r in range(c.num_reqs):
        blk = int(c.tables[r, 0])
        keys = -2.0 * u[:, None, :] + 0.3 * rng.standard_normal((H, b, d))
        c.k_pool[0][blk] = synth.f32_to_bf16_bits(keys.astype(np.float32))
    return c


def test_first_block_evicted_whole_every_row_moves():
    case = _max_shift_case()
    say("[gpu parity] maximum in-place shift: every head evicts its first block")
    run = run_case(case)
    b = case.geom.block_size
    first = run.kept[0][..., 0]
    assert np.all(first == b), first            # slots 0..b-1 gone: every kept row moved
    check_case(case, run)


def test_qwen3_8b_layer_full_size():
    """64 requests at budget 2048 (N_max=128, b=16, w=16), 8 KV / 32 query
    heads, d=128, bf16, pool of 16384 blocks: every output compared."""
    case = synth.case_qwen3_8b_layer()
    say("[gpu parity] qwen3-8b layer, 64 requests, budget 2048")
    run = run_case(case)
    stats = check_case(case, run)
    say(f"[gpu parity] qwen3-8b layer: ok {stats}")


# ---------------------------------------------------------------- decode alone

@pytest.mark.parametrize("dtype,d,b,G", [("bf16", 128, 16, 4), ("f32", 64, 32, 2), ("bf16", 64, 16, 8),
                                         ("f32", 128, 16, 1)])
def test_paged_decode_ragged_lengths(dtype, d, b, G):
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    H, max_blocks = 2, 40
    seqs = np.array([0, 1, b - 1, b, b + 1, 7 * b + 3, 16 * b, 16 * b + 1, 33 * b - 5,
                     max_blocks * b], dtype=np.int32)
    R = seqs.size
    c = _case("dec", 210, dtype=dtype, head_dim=d, block_size=b, num_reqs=R, num_kv_heads=H,
              num_q_heads=H * G, n_max=max_blocks, window=1, num_blocks=R * max_blocks + 3)
    say(f"[gpu parity] decode {dtype} d={d} b={b} G={G} seqs={seqs.tolist()}")
    dev = "cuda"
    kp, vp = to_tensor(c.k_pool[0], dev), to_tensor(c.v_pool[0], dev)
    cache = zp.KVCache([kp], [vp], H * G)
    tab = torch.from_numpy(c.tables).to(dev)
    seq_t = torch.from_numpy(seqs).to(dev)
    out = torch.full((R, H * G, d), float("nan"), device=dev)
    ws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, max_blocks), 16),
                     dtype=torch.uint8, device=dev)
    zp.paged_decode(cache, 0, to_tensor(c.q_new[0], dev), tab, seq_t, 1.0 / np.sqrt(d), out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.decode(c.k_pool[0], c.v_pool[0], c.q_new[0], c.tables, seqs, num_q_heads=H * G)
    assert np.isfinite(got).all()
    np.testing.assert_array_equal(got[0], 0.0)      # empty sequence -> zeros
    err = np.abs(got - want)
    assert err.max() <= DECODE_ATOL, err.max()


def test_empty_batches_do_nothing():
    """Zero requests: compression and decode enqueue nothing and change
    nothing (no tables, no freed blocks)."""
    import compressed_paged_kv_amd as zp
    from synth.device import to_numpy, to_tensor
    c = _case("empty", 221, num_reqs=1, n_max=4, num_blocks=8)
    dev = "cuda"
    say("[gpu parity] empty batches")
    kp, vp = to_tensor(c.k_pool[0], dev), to_tensor(c.v_pool[0], dev)
    cache = zp.KVCache([kp], [vp], c.geom.num_q_heads)
    pool = zp.BlockPool.from_refcounts(c.refcounts)
    before = pool.refcounts()
    tables = np.zeros((0, c.n_max), dtype=np.int32)
    wq = [torch.empty((0, c.window, c.geom.num_q_heads, c.geom.head_dim), dtype=kp.dtype,
                      device=dev)]
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    freed = zp.compress(cache, pool, c.n_max, c.window, tables, wq, ws)
    assert freed.size == 0
    out = torch.empty((0, c.geom.num_q_heads, c.geom.head_dim), device=dev)
    zp.paged_decode(cache, 0, torch.empty((0, c.geom.num_q_heads, c.geom.head_dim),
                                          dtype=kp.dtype, device=dev),
                    torch.zeros((0, c.n_max), dtype=torch.int32, device=dev),
                    torch.zeros(0, dtype=torch.int32, device=dev), 0.125, out, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pool.refcounts(), before)
    np.testing.assert_array_equal(to_numpy(kp), c.k_pool[0])


def test_decode_skips_table_entries_outside_the_pool():
    """A block id outside [0, num_blocks) (negative or too large) is skipped
    by the kernel's own guard: the output is the attention over the other
    blocks' slots, which the oracle gets from the table without them (the
    attention is a sum over the set of slots, so their order is free).  A
    request whose every entry is outside the pool attends over nothing: its
    output is 0 and its log-sum-exp -inf, as for an empty request.  Three
    requests alone split their 20-block lists over three workgroups each;
    the same requests repeated 100 times fill the GPU without splits."""
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    b, H, Hq, d, nb = 16, 2, 8, 128, 20
    c = _case("guard", 222, num_reqs=3, num_kv_heads=H, num_q_heads=Hq, head_dim=d,
              block_size=b, n_max=nb, window=1, num_blocks=64)
    say("[gpu parity] decode with table entries outside the pool")
    dev = "cuda"
    kp, vp = to_tensor(c.k_pool[0], dev), to_tensor(c.v_pool[0], dev)
    cache = zp.KVCache([kp], [vp], Hq)
    tab = c.tables.copy()
    tab[0, 1] = 64 + 5          # past the pool
    tab[1, 3] = -7              # negative
    tab[2, :] = np.where(np.arange(nb) % 2 == 0, -1 - np.arange(nb), 64 + np.arange(nb))
    tab[2, 5] = 1 << 30
    seq = np.array([17 * b + 7, 12 * b, nb * b], dtype=np.int32)
    # request 0: blocks 0, 2..17 (the last holds 7 slots); request 1: blocks 0..2, 4..11
    keep0 = np.array([c.tables[0, i] for i in [0] + list(range(2, 18))], dtype=np.int32)
    keep1 = np.array([c.tables[1, i] for i in [0, 1, 2] + list(range(4, 12))], dtype=np.int32)
    want0 = oracle.decode(c.k_pool[0], c.v_pool[0], c.q_new[0][:1], keep0[None],
                          np.array([16 * b + 7], dtype=np.int32), num_q_heads=Hq)
    want1 = oracle.decode(c.k_pool[0], c.v_pool[0], c.q_new[0][1:2], keep1[None],
                          np.array([11 * b], dtype=np.int32), num_q_heads=Hq)
    lse0 = oracle.decode_lse(c.k_pool[0], c.q_new[0][:1], keep0[None],
                             np.array([16 * b + 7], dtype=np.int32), num_q_heads=Hq)
    q = to_tensor(c.q_new[0], dev)
    for reps in (1, 100):
        R = 3 * reps
        qs = q.repeat(reps, 1, 1).contiguous()
        tabs = np.ascontiguousarray(np.tile(tab, (reps, 1)))
        seqs = np.ascontiguousarray(np.tile(seq, reps))
        out = torch.full((R, Hq, d), float("nan"), device=dev)
        lse = torch.full((R, Hq), float("nan"), device=dev)
        ws_bytes = zp.paged_decode_workspace_bytes(cache, R, nb)
        assert (ws_bytes > 0) == (reps == 1), ws_bytes      # split only when alone
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        zp.paged_decode(cache, 0, qs, torch.from_numpy(tabs).to(dev),
                        torch.from_numpy(seqs).to(dev), 1.0 / np.sqrt(d), out, ws, lse_out=lse)
        torch.cuda.synchronize()
        got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
        for k in range(reps):
            assert np.abs(got[3 * k] - want0[0]).max() <= DECODE_ATOL
            assert np.abs(got[3 * k + 1] - want1[0]).max() <= DECODE_ATOL
            np.testing.assert_array_equal(got[3 * k + 2], 0.0)
            assert np.all(np.isneginf(got_lse[3 * k + 2])), got_lse[3 * k + 2]
            assert np.abs(got_lse[3 * k] - lse0[0]).max() <= 1e-4 * max(1.0, np.abs(lse0).max())


def test_append_then_decode_one_token():
    """A request of length 1: the appended row is the only key, so the output
    equals the appended value exactly (softmax over one slot)."""
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    c = _case("app", 211, dtype="f32", num_reqs=3, n_max=4, num_blocks=16, head_dim=64)
    dev = "cuda"
    kp, vp = to_tensor(c.k_pool[0], dev), to_tensor(c.v_pool[0], dev)
    cache = zp.KVCache([kp], [vp], 4)
    slot = (c.tables[:, 0] * 16).astype(np.int32)
    slot[1] = -1                                     # skipped
    zp.append_kv(cache, 0, to_tensor(c.k_new[0], dev), to_tensor(c.v_new[0], dev),
                 torch.from_numpy(slot).to(dev))
    out = torch.empty((3, 4, 64), device=dev)
    zp.paged_decode(cache, 0, to_tensor(c.q_new[0], dev), torch.from_numpy(c.tables).to(dev),
                    torch.ones(3, dtype=torch.int32, device=dev), 0.125, out, None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in (0, 2):
        for hq in range(4):
            np.testing.assert_array_equal(got[r, hq], c.v_new[0][r, hq // 2])
    blk = int(c.tables[1, 0])
    np.testing.assert_array_equal(kp[blk].cpu().numpy(), c.k_pool[0][blk])


# ---------------------------------------------------------------- prefix-keeping compression

def test_keep_prefix_leaves_a_clean_shared_prefix_shared():
    """Exact ties put every eviction at the highest candidate slots, past a
    3-block prefix shared by 4 requests: zp_compress_keep_prefix keeps the
    prefix blocks in every table (still shared, bytes unchanged, nothing
    freed) and matches the oracle's prefix-keeping plan and compaction."""
    c = _case("kp", 240, num_reqs=4, num_layers=2, n_max=12, num_blocks=80,
              shared_prefix_blocks=3)
    R, H, b, d = c.num_reqs, c.geom.num_kv_heads, c.geom.block_size, c.geom.head_dim
    T = c.n_max * b
    K = np.zeros((R, H, T, d))
    for j in range(T):
        K[:, :, j, j % b] = 1.0 + (j % 3)
    for l in range(2):
        c.k_pool[l] = synth.pool_from_logical(K, c.tables, c.geom.num_blocks, "bf16")
        c.window_q[l] = np.zeros_like(c.window_q[l])
    say("[gpu parity] keep-prefix: 4 requests, 3 shared blocks, exact ties")
    run = run_case(c, keep_prefix=True)
    prefix = c.tables[0, :3]
    assert np.all(run.tables[:, :3] == prefix) and run.freed.size == 0
    assert all(run.refcounts[x] == R for x in prefix)
    check_case(c, run, keep_prefix=True)


@pytest.mark.parametrize("name", ["shared_prefix_2layers", "over_cap_prefix_2layers",
                                  "mixed_counts_prefix_2layers"])
def test_keep_prefix_matches_oracle_on_random_prefixes(name):
    case = CASES[name]()
    say(f"[gpu parity] keep-prefix on {name}")
    run = run_case(case, keep_prefix=True)
    stats = check_case(case, run, keep_prefix=True)
    say(f"[gpu parity] keep-prefix {name}: ok {stats}")


def _random_configs(n, seed):
    """Seeded random shapes inside the host's limits, including the corner
    n_max = 2 (one target block plus the reserved one; with w = b every
    candidate is evicted)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        b = int(rng.choice([16, 32]))
        w = int(rng.integers(1, b + 1))
        G = int(rng.choice([1, 2, 4, 8]))
        H = int(rng.integers(1, 3))
        n_max = 2 if len(out) < 3 else int(rng.integers(2, 33))
        n_src = n_max + int(rng.integers(0, 4)) if rng.random() < 0.3 else n_max
        if G * w > 128 or (G * w > 64 and n_src * b > 4096):
            continue
        if (n_src - n_max + 1) * b > 1024:
            continue
        R = int(rng.integers(1, 4))
        L = int(rng.integers(1, 3))
        P = int(rng.integers(0, min(n_max - 1, 3) + 1)) if R > 1 and rng.random() < 0.4 else 0
        nb = P + R * (n_src - P) + R * n_max + 4
        out.append(dict(num_reqs=R, num_layers=L, num_kv_heads=H, num_q_heads=H * G,
                        head_dim=int(rng.choice([64, 128])), block_size=b, n_max=n_max,
                        window=w, num_blocks=nb, dtype=str(rng.choice(["bf16", "f32"])),
                        shared_prefix_blocks=P, n_src=n_src))
    # n_max = 2 with w = b: no candidate survives (K_sel = 0)
    out.append(dict(num_reqs=2, num_layers=1, num_kv_heads=2, num_q_heads=4, head_dim=128,
                    block_size=16, n_max=2, window=16, num_blocks=12, dtype="bf16",
                    shared_prefix_blocks=0, n_src=2))
    return out


@pytest.mark.parametrize("i,cfg", list(enumerate(_random_configs(24, 4242))))
def test_random_shapes_match_oracle(i, cfg):
    case = synth.make_case(f"rand{i}", 5000 + i, **cfg)
    say(f"[gpu parity] random shape {i}: {cfg}")
    run = run_case(case)
    check_case(case, run)


def _random_mixed_configs(n, seed):
    """Seeded calls over requests holding different block counts, inside
    the host's limits for the largest of them."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        b = int(rng.choice([16, 32]))
        w = int(rng.integers(1, b + 1))
        G = int(rng.choice([1, 2, 4, 8]))
        H = int(rng.integers(1, 3))
        n_max = int(rng.integers(2, 25))
        R = int(rng.integers(2, 5))
        counts = [n_max + (int(rng.integers(0, 8)) if rng.random() < 0.6 else 0) for _ in range(R)]
        if max(counts) == n_max:
            counts[int(rng.integers(0, R))] += 1
        if G * w > 128 or (G * w > 64 and max(counts) * b > 4096):
            continue
        if (max(counts) - n_max + 1) * b > 1024:
            continue
        P = int(rng.integers(0, min(n_max - 1, 3) + 1)) if rng.random() < 0.4 else 0
        nb = P + sum(c - P for c in counts) + R * n_max + 4
        out.append(dict(num_reqs=R, num_layers=int(rng.integers(1, 3)), num_kv_heads=H,
                        num_q_heads=H * G, head_dim=int(rng.choice([64, 128])), block_size=b,
                        n_max=n_max, window=w, num_blocks=nb,
                        dtype=str(rng.choice(["bf16", "f32"])), shared_prefix_blocks=P,
                        n_src=counts))
    return out


@pytest.mark.parametrize("i,cfg", list(enumerate(_random_mixed_configs(10, 5151))))
def test_random_mixed_block_counts_match_oracle(i, cfg):
    case = synth.make_case(f"mixed{i}", 5200 + i, **cfg)
    say(f"[gpu parity] random mixed counts {i}: {cfg}")
    run = run_case(case)
    check_case(case, run)


def _random_decode_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        b, d = int(rng.choice([16, 32])), int(rng.choice([64, 128]))
        G, H = int(rng.choice([1, 2, 4, 8])), int(rng.integers(1, 4))
        R, mb = int(rng.integers(1, 40)), int(rng.integers(1, 70))
        seqs = rng.integers(0, mb * b + 1, size=R).astype(np.int32)
        out.append((b, d, G, H, R, mb, str(rng.choice(["bf16", "f32"])), seqs))
    return out


@pytest.mark.parametrize("i,cfg", list(enumerate(_random_decode_configs(20, 31))))
def test_random_decode_shapes_match_oracle(i, cfg):
    """Seeded random batches (with and without splits of the block list):
    output and log-sum-exp against the oracle."""
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    b, d, G, H, R, mb, dtype, seqs = cfg
    c = synth.make_case(f"dec{i}", 70000 + i, num_reqs=R, num_layers=1, num_kv_heads=H,
                        num_q_heads=H * G, head_dim=d, block_size=b, n_max=mb, window=1,
                        num_blocks=R * mb + 3, dtype=dtype)
    say(f"[gpu parity] random decode {i}: R={R} H={H} G={G} d={d} b={b} max_blocks={mb} {dtype}")
    dev = "cuda"
    kp, vp = to_tensor(c.k_pool[0], dev), to_tensor(c.v_pool[0], dev)
    cache = zp.KVCache([kp], [vp], H * G)
    out = torch.full((R, H * G, d), float("nan"), device=dev)
    lse = torch.full((R, H * G), float("nan"), device=dev)
    ws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, mb), 16), dtype=torch.uint8,
                     device=dev)
    zp.paged_decode(cache, 0, to_tensor(c.q_new[0], dev), torch.from_numpy(c.tables).to(dev),
                    torch.from_numpy(seqs).to(dev), 1.0 / np.sqrt(d), out, ws, lse_out=lse)
    torch.cuda.synchronize()
    want = oracle.decode(c.k_pool[0], c.v_pool[0], c.q_new[0], c.tables, seqs, num_q_heads=H * G)
    want_lse = oracle.decode_lse(c.k_pool[0], c.q_new[0], c.tables, seqs, num_q_heads=H * G)
    got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(got).all() and np.abs(got - want).max() <= DECODE_ATOL
    fin = np.isfinite(want_lse)
    np.testing.assert_array_equal(np.isfinite(got_lse), fin)      # -inf for empty requests
    if fin.any():
        assert np.abs(got_lse[fin] - want_lse[fin]).max() <= 1e-4 * max(1.0, np.abs(want_lse[fin]).max())


def _fused_equals_standalone(case, want_k_cached):
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    g = case.geom
    assert np.all(case.refcounts <= 1), "the case must have no shared blocks"
    cache = zp.KVCache([to_tensor(x, "cuda") for x in case.k_pool[:1]] * g.num_layers,
                       [to_tensor(x, "cuda") for x in case.v_pool[:1]] * g.num_layers,
                       g.num_q_heads)
    info = zp.compress_query(cache, case.num_reqs, case.n_max, case.window, n_src=case.n_src)
    say(f"[gpu parity]   launch: {info}")
    assert info["k_cached"] == want_k_cached, info
    del cache
    fused = run_case(case, decode=False)
    split = run_case(case, decode=False, keep_prefix=True)
    np.testing.assert_array_equal(fused.tables, split.tables)
    np.testing.assert_array_equal(fused.refcounts, split.refcounts)
    np.testing.assert_array_equal(fused.kept, split.kept)
    for a, b in zip(fused.k_pool + fused.v_pool, split.k_pool + split.v_pool):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                              np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("name", ["bf16_d128_b16_ragged", "bf16_d64_b32_rows128",
                                  "f32_d128_b32_w5", "over_cap_bf16_3_extra",
                                  "mixed_counts_b32_rows128", "mixed_counts_f32_d64"])
def test_fused_compaction_equals_the_standalone_kernel(name):
    """Without shared blocks the prefix-keeping call makes the same plan as
    the plain one, but runs the selection and the compaction as two kernels
    (its plan waits for the selection), while the plain call compacts inside
    the scoring kernel: the pools and tables must come out bit-identical.
    These small calls have every unit resident at once, so the fused
    compaction loads K normally."""
    case = CASES[name]()
    say(f"[gpu parity] fused vs standalone compaction: {name}")
    _fused_equals_standalone(case, want_k_cached=1)


def test_fused_compaction_streaming_k_equals_the_standalone_kernel():
    """The other branch of the fused compaction: a call with more units than
    the GPU holds at once (sized from the device's own resident count for
    this shape) streams K; pools and tables bit-identical to the two-kernel
    path, and the kept lists to the oracle's rule on the GPU's scores."""
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    kw = dict(num_layers=3, num_kv_heads=8, num_q_heads=16, head_dim=64, n_max=6)
    probe = _case("m6probe", 226, num_reqs=1, num_blocks=8, **kw)
    cache = zp.KVCache([to_tensor(probe.k_pool[0], "cuda")] * 3,
                       [to_tensor(probe.v_pool[0], "cuda")] * 3, 16)
    info = zp.compress_query(cache, 1, 6, 16)
    del cache
    fit = info["resident_per_cu"] * info["compute_units"]
    R = fit // (3 * 8) + 1                 # one more request than fits at once
    say(f"[gpu parity] fused vs standalone, streamed K: {info}, {R} requests "
        f"({3 * 8 * R} units for {fit} resident)")
    case = _case("m6", 226, num_reqs=R, num_blocks=R * 6 + 8, **kw)
    _fused_equals_standalone(case, want_k_cached=0)
    check_case(case, run_case(case))


@pytest.mark.parametrize("name,keep_prefix", [
    ("tiny", False),                          # in place: nothing uploaded
    ("bf16_d128_b16_ragged", False),
    ("shared_prefix_2layers", False),         # re-targets: the target table is uploaded
    ("over_cap_prefix_2layers", False),       # past the cap, shared prefix
    ("over_cap_bf16_3_extra", False),         # past the cap, in place
    ("layers_50_two_launches", False),        # two launches of layer chunks
    ("shared_prefix_2layers", True),          # prefix keeping with device sources
    ("bf16_d128_b16_ragged", True),
    ("mixed_counts_prefix_2layers", False),   # requests holding different block counts
    ("mixed_counts_prefix_2layers", True),
    ("mixed_counts_f32_d64", False),
])
def test_device_tables_equal_the_uploaded_tables(name, keep_prefix):
    """zp_compress_ex with the caller's device copy of the tables: the same
    pools, tables, survivor lists and decode outputs, bit for bit, as the
    call that uploads its tables, and the oracle's results."""
    case = CASES[name]()
    say(f"[gpu parity] device tables: {name}, keep_prefix={keep_prefix}")
    up = run_case(case, keep_prefix=keep_prefix)
    dv = run_case(case, keep_prefix=keep_prefix, device_tables=True)
    np.testing.assert_array_equal(up.tables, dv.tables)
    np.testing.assert_array_equal(up.refcounts, dv.refcounts)
    np.testing.assert_array_equal(np.sort(up.freed), np.sort(dv.freed))
    np.testing.assert_array_equal(up.kept, dv.kept)
    for a, b in zip(up.appended_k + up.appended_v, dv.appended_k + dv.appended_v):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                              np.ascontiguousarray(b).view(np.uint8))
    np.testing.assert_array_equal(up.out.view(np.uint32), dv.out.view(np.uint32))
    check_case(case, dv, keep_prefix=keep_prefix)


def test_debug_poison_changes_nothing_a_correct_reader_sees():
    """With ZP_DEBUG_POISON the compression leaves NaN in the blocks it frees
    and in every slot of the reserved blocks; everything else -- tables,
    compacted targets, the appended token and the decode output -- is bit
    for bit what the same call gives without it."""
    import compressed_paged_kv_amd as zp
    case = CASES["shared_prefix_2layers"]()      # 4 requests re-target a shared 3-block prefix
    say("[gpu parity] debug poison on the shared-prefix case")
    before = zp.debug_flags()
    plain = run_case(case, decode=False)
    try:
        zp.set_debug_flags(zp.ZP_DEBUG_POISON)
        poisoned = run_case(case, decode=False)
    finally:
        zp.set_debug_flags(before)
    np.testing.assert_array_equal(plain.tables, poisoned.tables)
    freed = np.asarray(poisoned.freed)
    assert freed.size == 3
    reserved = poisoned.tables[:, case.n_max - 1]
    bad = set(freed.tolist()) | set(reserved.tolist())
    for a, b in zip(plain.k_pool + plain.v_pool, poisoned.k_pool + poisoned.v_pool):
        fa = a.astype(np.float32) if a.dtype == np.float32 else synth.bf16_bits_to_f32(a)
        fb = b.astype(np.float32) if b.dtype == np.float32 else synth.bf16_bits_to_f32(b)
        for blk in range(a.shape[0]):
            if blk in bad:
                assert np.isnan(fb[blk]).all(), blk
            else:
                assert np.array_equal(a[blk].view(np.uint8), b[blk].view(np.uint8)), blk
    # the decode after the append reads only slots up to the new length
    zp.set_debug_flags(zp.ZP_DEBUG_POISON)
    try:
        dec = run_case(case)
    finally:
        zp.set_debug_flags(before)
    ref = run_case(case)
    np.testing.assert_array_equal(dec.out.view(np.uint32), ref.out.view(np.uint32))


def test_validate_rejects_a_device_table_that_differs():
    """ZP_DEBUG_VALIDATE: zp_compress_ex reads the device copy back and
    rejects a call whose copy differs from the host tables, changing nothing
    (tables, reference counts, pools)."""
    import compressed_paged_kv_amd as zp
    from synth.device import to_numpy, to_tensor
    case = CASES["bf16_d128_b16_ragged"]()
    g = case.geom
    say("[gpu parity] validate device tables")
    kp = [to_tensor(x, "cuda") for x in case.k_pool]
    vp = [to_tensor(x, "cuda") for x in case.v_pool]
    wq = [to_tensor(x, "cuda") for x in case.window_q]
    cache = zp.KVCache(kp, vp, g.num_q_heads)
    pool = zp.BlockPool.from_refcounts(case.refcounts)
    ws = torch.empty(zp.compress_workspace_bytes(cache, case.num_reqs, case.n_max, case.window),
                     dtype=torch.uint8, device="cuda")
    wrong = case.tables.copy()
    wrong[1, 5], wrong[1, 6] = wrong[1, 6], wrong[1, 5]
    before = zp.debug_flags()
    zp.set_debug_flags(zp.ZP_DEBUG_VALIDATE)
    try:
        tables = case.tables.copy()
        with pytest.raises(zp.ZpError) as e:
            zp.compress(cache, pool, case.n_max, case.window, tables, wq, ws,
                        device_tables=torch.from_numpy(wrong).to("cuda"))
        assert e.value.status == zp.ZP_ERR_INVALID and "device_tables differ" in str(e.value)
        np.testing.assert_array_equal(tables, case.tables)
        np.testing.assert_array_equal(pool.refcounts(), case.refcounts)
        torch.cuda.synchronize()
        for l in range(g.num_layers):
            assert np.array_equal(to_numpy(kp[l]).view(np.uint8), case.k_pool[l].view(np.uint8))
        # the matching copy goes through
        zp.compress(cache, pool, case.n_max, case.window, tables, wq, ws,
                    device_tables=torch.from_numpy(np.ascontiguousarray(case.tables)).to("cuda"))
        torch.cuda.synchronize()
    finally:
        zp.set_debug_flags(before)
    pool.sync()


@pytest.mark.parametrize("dtype,d,b,G,R,mb", [("bf16", 128, 16, 4, 3, 40),    # split lists
                                              ("bf16", 128, 16, 4, 300, 9),   # no split
                                              ("f32", 64, 32, 8, 5, 12)])
def test_decode_bfloat16_output_is_the_rounded_float32_output(dtype, d, b, G, R, mb):
    """zp_paged_decode_ex with out_dtype ZP_BF16: every element is the
    float32 result of the same call rounded to nearest even (bit for bit),
    log-sum-exp unchanged."""
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    H = 2
    c = synth.make_case("dec_bf16", 6100 + R, num_reqs=R, num_layers=1, num_kv_heads=H,
                        num_q_heads=H * G, head_dim=d, block_size=b, n_max=mb, window=1,
                        num_blocks=R * mb + 3, dtype=dtype)
    say(f"[gpu parity] bf16 decode output {dtype} d={d} b={b} G={G} R={R} max_blocks={mb}")
    rng = np.random.default_rng(61)
    seqs = rng.integers(0, mb * b + 1, size=R).astype(np.int32)
    dev = "cuda"
    kp, vp = to_tensor(c.k_pool[0], dev), to_tensor(c.v_pool[0], dev)
    cache = zp.KVCache([kp], [vp], H * G)
    q, tab = to_tensor(c.q_new[0], dev), torch.from_numpy(c.tables).to(dev)
    seq_t = torch.from_numpy(seqs).to(dev)
    ws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, mb), 16), dtype=torch.uint8,
                     device=dev)
    o32 = torch.full((R, H * G, d), float("nan"), device=dev)
    o16 = torch.full((R, H * G, d), float("nan"), dtype=torch.bfloat16, device=dev)
    l32 = torch.full((R, H * G), float("nan"), device=dev)
    l16 = torch.full((R, H * G), float("nan"), device=dev)
    zp.paged_decode(cache, 0, q, tab, seq_t, 1.0 / np.sqrt(d), o32, ws, lse_out=l32)
    zp.paged_decode(cache, 0, q, tab, seq_t, 1.0 / np.sqrt(d), o16, ws, lse_out=l16)
    torch.cuda.synchronize()
    want = synth.f32_to_bf16_bits(o32.cpu().numpy())
    got = o16.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(l16.cpu().numpy().view(np.uint32), l32.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("name,recorded,keep_prefix", [
    ("bf16_d128_b16_ragged", False, False),
    ("bf16_d64_b32_rows128", False, False),   # two row groups
    ("shared_prefix_2layers", False, False),  # re-targets
    ("shared_prefix_2layers", False, True),   # prefix keeping: the selection kernel alone
    ("over_cap_bf16_3_extra", True, False),   # recorded normalisers, past the cap
    ("mixed_counts_prefix_2layers", True, False),
    ("f32_d128_b32_w5", True, False),
])
def test_window_rows_read_in_place_from_query_slots(name, recorded, keep_prefix):
    """zp_compress_ex with window_slots: the window rows (and recorded
    normalisers) read in place from query-slot stores, each request at a
    permuted slot and every other slot NaN, give bit for bit the results of
    the call that takes them gathered per request, and the oracle's."""
    case = CASES[name]()
    say(f"[gpu parity] window rows from query slots: {name}, recorded={recorded}, "
        f"keep_prefix={keep_prefix}")
    ref = run_case(case, recorded_lse=recorded, keep_prefix=keep_prefix)
    got = run_case(case, recorded_lse=recorded, keep_prefix=keep_prefix, slot_store=77)
    np.testing.assert_array_equal(ref.tables, got.tables)
    np.testing.assert_array_equal(ref.refcounts, got.refcounts)
    np.testing.assert_array_equal(ref.kept, got.kept)
    for a, b in ((ref.A, got.A), (ref.R, got.R), (ref.s, got.s)):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    for a, b in zip(ref.appended_k + ref.appended_v, got.appended_k + got.appended_v):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                              np.ascontiguousarray(b).view(np.uint8))
    np.testing.assert_array_equal(ref.out.view(np.uint32), got.out.view(np.uint32))
    check_case(case, got, keep_prefix=keep_prefix)


@pytest.mark.parametrize("name,keep_prefix,recorded", [
    ("bf16_d128_b16_ragged", False, False),   # fused: start, pass 1, pass 2, selection, compaction
    ("bf16_d64_b32_rows128", False, True),    # two row groups, recorded normalisers (no pass 1)
    ("shared_prefix_2layers", True, False),   # the selection-only kernel
])
def test_phase_times_are_stamped_in_order_and_change_nothing(name, keep_prefix, recorded):
    """debug phase_times: every unit's five wall-clock stamps are set and
    non-decreasing, within the call, and asking for them leaves every other
    result bit-identical."""
    import compressed_paged_kv_amd as zp
    case = CASES[name]()
    say(f"[gpu parity] phase times: {name}, keep_prefix={keep_prefix}, recorded={recorded}")
    ref = run_case(case, decode=False, keep_prefix=keep_prefix, recorded_lse=recorded)
    got = run_case(case, decode=False, keep_prefix=keep_prefix, recorded_lse=recorded,
                   phase_times=True)
    np.testing.assert_array_equal(ref.tables, got.tables)
    np.testing.assert_array_equal(ref.kept, got.kept)
    for a, b in zip(ref.k_pool + ref.v_pool, got.k_pool + got.v_pool):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                              np.ascontiguousarray(b).view(np.uint8))
    for a, b in ((ref.A, got.A), (ref.R, got.R), (ref.s, got.s)):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    t = got.times.reshape(-1, 5)
    assert (t > 0).all(), "a unit left a stamp unset"
    assert (np.diff(t, axis=1) >= 0).all(), "stamps out of order"
    from synth.device import to_tensor
    g = case.geom
    cache = zp.KVCache([to_tensor(case.k_pool[0], "cuda")] * g.num_layers,
                       [to_tensor(case.v_pool[0], "cuda")] * g.num_layers, g.num_q_heads)
    khz = zp.compress_query(cache, case.num_reqs, case.n_max, case.window,
                            n_src=case.n_src)["wall_clock_khz"]
    assert khz > 0
    span_ms = (t[:, 4].max() - t[:, 0].min()) / khz
    say(f"[gpu parity]   clock {khz} kHz, span {span_ms * 1e3:.1f} us")
    assert span_ms < 1000.0


def _random_feature_configs(n, seed):
    """Seeded shapes (uniform or mixed block counts, optional shared prefix)
    each with a seeded choice of the call's options."""
    rng = np.random.default_rng(seed)
    out = []
    shapes = _random_mixed_configs(n, seed + 1) + _random_configs(n, seed + 2)
    for i in range(n):
        cfg = dict(shapes[rng.integers(0, len(shapes))])
        opts = dict(recorded_lse=bool(rng.random() < 0.5), keep_prefix=bool(rng.random() < 0.3),
                    device_tables=bool(rng.random() < 0.5),
                    slot_store=int(rng.integers(1, 1000)) if rng.random() < 0.5 else None)
        out.append((cfg, opts))
    return out


@pytest.mark.parametrize("i,cfg,opts", [(i, c, o) for i, (c, o) in
                                         enumerate(_random_feature_configs(16, 6161))])
def test_random_feature_combinations_match_oracle(i, cfg, opts):
    """Random shapes with a random mix of the call's options (per-request
    block counts, device tables, prefix keeping, recorded normalisers, window
    rows read in place from query slots), each against the oracle."""
    case = synth.make_case(f"combo{i}", 5400 + i, **cfg)
    say(f"[gpu parity] feature combination {i}: {cfg} {opts}")
    run = run_case(case, **opts)
    check_case(case, run, keep_prefix=opts["keep_prefix"])

