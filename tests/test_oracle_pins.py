"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, a worked example, a
library routine, brute force on tiny inputs, or an invariant the pages fix,
chosen so that a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one in the causal window, a reversed tie rule)
fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac(tok):
    return float(Fraction(tok))


def _read_golden(name):
    items = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, vals = line.partition(":")
            items[key.strip()] = vals.split()
    return items


def _tiny_case(rng, *, R=2, H=2, Hq=4, d=8, b=4, n_max=5, w=3, pool=24, dtype="f32",
               K=None, Q=None):
    """Random logical keys/queries scattered through a permuted block table."""
    T = n_max * b
    tables = rng.permutation(pool)[: R * n_max].astype(np.int32).reshape(R, n_max)
    if K is None:
        K = rng.standard_normal((R, H, T, d))
    if Q is None:
        Q = rng.standard_normal((R, w, Hq, d))
    kpool = synth.pool_from_logical(K, tables, pool, dtype)
    qstore = Q.astype(np.float32) if dtype == "f32" else synth.f32_to_bf16_bits(Q.astype(np.float32))
    return tables, kpool, qstore, K, Q


# ---------------------------------------------------------------- worked example

def test_worked_example_closed_form():
    g = _read_golden("worked_example_q0.txt")
    keys = np.array([float(x) for x in g["keys"]]).reshape(12, 2)
    table = np.array([int(x) for x in g["table_before"]], dtype=np.int32)[None, :]
    rc = np.array([int(x) for x in g["refcounts_before"]], dtype=np.int32)
    kpool = synth.pool_from_logical(keys[None, None], table, 8, "f32")
    wq = np.zeros((1, 2, 1, 2), dtype=np.float32)

    p = oracle.plan(rc, table, 3)
    assert p.status == oracle.OK
    assert p.tables[0].tolist() == [int(x) for x in g["table_after"]]
    assert p.refcounts.tolist() == [int(x) for x in g["refcounts_after"]]
    assert p.dst[0].tolist() == [int(x) for x in g["dst"]]
    assert p.freed.tolist() == [int(x) for x in g.get("freed", [])]

    A, R, s = oracle.scores(kpool, wq, p.src, num_kv_heads=1, num_q_heads=1, head_dim=2,
                            block_size=4, n_max=3, window=2)
    np.testing.assert_allclose(A[0, 0], [_frac(x) for x in g["A"]], rtol=1e-15, atol=0)
    np.testing.assert_allclose(R[0, 0], [_frac(x) for x in g["R"]], rtol=0, atol=1e-15)
    a0 = _frac("23/264")
    np.testing.assert_allclose(s[0, 0, :10] / a0, [_frac(x) for x in g["s_over_A"]], rtol=1e-14)
    # the tie s3 == s9 must be exact for the tie rule to decide it
    assert s[0, 0, 3] == s[0, 0, 9]
    kept = oracle.select(s, 2, 6)
    assert kept[0, 0].tolist() == [int(x) for x in g["kept"]]

    new = oracle.compact(kpool, p.src, p.dst, kept[0:1], n_max=3)
    got = bf.logical_rows(new, p.tables[0], 0, 8)
    np.testing.assert_array_equal(got, keys[kept[0, 0]])


# ---------------------------------------------------------------- importance A

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_importance_sums_to_one(dtype):
    rng = np.random.default_rng(7)
    tables, kpool, q, _, _ = _tiny_case(rng, dtype=dtype)
    A, _, _ = oracle.scores(kpool, q, tables, num_kv_heads=2, num_q_heads=4, head_dim=8,
                            block_size=4, n_max=5, window=3)
    np.testing.assert_allclose(A.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    assert (A > 0).all()


def test_importance_zero_query_closed_form():
    rng = np.random.default_rng(8)
    w, b, n_max = 3, 4, 5
    T = n_max * b
    Q = np.zeros((2, w, 4, 8))
    tables, kpool, q, _, _ = _tiny_case(rng, Q=Q)
    A, _, _ = oracle.scores(kpool, q, tables, num_kv_heads=2, num_q_heads=4, head_dim=8,
                            block_size=b, n_max=n_max, window=w)
    p = T - w + np.arange(w)
    want = np.array([sum(1.0 / (pi + 1) for pi in p if pi >= j) for j in range(T)]) / w
    np.testing.assert_allclose(A, np.broadcast_to(want, A.shape), rtol=1e-14)


@pytest.mark.parametrize("G,w", [(1, 1), (2, 3), (4, 4)])
def test_importance_matches_dense_scipy_softmax(G, w):
    rng = np.random.default_rng(9 + G)
    H, d, b, n_max = 2, 8, 4, 6
    tables, kpool, q, K, Q = _tiny_case(rng, H=H, Hq=H * G, d=d, b=b, n_max=n_max, w=w)
    A, _, _ = oracle.scores(kpool, q, tables, num_kv_heads=H, num_q_heads=H * G, head_dim=d,
                            block_size=b, n_max=n_max, window=w)
    Qf = q.astype(np.float64)
    for r in range(2):
        for h in range(H):
            Kl = bf.logical_rows(kpool, tables[r], h, n_max * b)
            Qw = Qf[r][:, h * G:(h + 1) * G, :]          # [w][G][d]
            np.testing.assert_allclose(A[r, h], bf.importance_dense(Kl, Qw), rtol=1e-12)


def test_importance_planted_key_dominates():
    rng = np.random.default_rng(11)
    R, H, G, d, b, n_max, w = 1, 1, 2, 16, 4, 6, 3
    T = n_max * b
    Q = rng.standard_normal((R, w, H * G, d))
    K = rng.standard_normal((R, H, T, d))
    planted = 9
    direction = Q[0].reshape(-1, d).sum(axis=0)
    K[0, 0, planted] = 4.0 * direction / np.linalg.norm(direction) * np.sqrt(d)
    tables, kpool, q, _, _ = _tiny_case(rng, R=R, H=H, Hq=H * G, d=d, b=b, n_max=n_max, w=w,
                                        K=K, Q=Q)
    A, _, _ = oracle.scores(kpool, q, tables, num_kv_heads=H, num_q_heads=H * G, head_dim=d,
                            block_size=b, n_max=n_max, window=w)
    assert int(np.argmax(A[0, 0])) == planted


def test_importance_reads_through_table_and_group():
    """Swapping two physical blocks and their table entries changes nothing;
    swapping the query heads of two KV groups swaps the groups' scores."""
    rng = np.random.default_rng(12)
    tables, kpool, q, _, _ = _tiny_case(rng)
    kw = dict(num_kv_heads=2, num_q_heads=4, head_dim=8, block_size=4, n_max=5, window=3)
    A1, R1, _ = oracle.scores(kpool, q, tables, **kw)
    a, c = int(tables[0, 1]), int(tables[1, 3])
    kp2 = kpool.copy()
    kp2[[a, c]] = kpool[[c, a]]
    t2 = tables.copy()
    t2[0, 1], t2[1, 3] = c, a
    A2, R2, _ = oracle.scores(kp2, q, t2, **kw)
    np.testing.assert_array_equal(A1, A2)
    np.testing.assert_array_equal(R1, R2)
    # query heads 0,1 belong to KV head 0 and 2,3 to KV head 1
    q2 = q[:, :, [2, 3, 0, 1], :].copy()
    kp3 = kpool[:, [1, 0]].copy()
    A3, _, _ = oracle.scores(kp3, q2, tables, **kw)
    np.testing.assert_allclose(A3[:, [1, 0]], A1, rtol=1e-14)


# ---------------------------------------------------------------- redundancy R

def _as_stored(x):
    """The values a float32 pool actually holds, as float64."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _lrs(K, b, n_max, d):
    R, H, T, _ = K.shape
    tables = np.arange(R * n_max, dtype=np.int32).reshape(R, n_max)
    kpool = synth.pool_from_logical(K, tables, R * n_max, "f32")
    q = np.zeros((R, 1, H, d), dtype=np.float32)
    _, Rr, _ = oracle.scores(kpool, q, tables, num_kv_heads=H, num_q_heads=H, head_dim=d,
                             block_size=b, n_max=n_max, window=1)
    return Rr


def test_lrs_special_cases():
    d, b = 8, 4
    rng = np.random.default_rng(13)
    v = rng.standard_normal(d)
    # block 0: identical keys -> 1; block 1: scaled basis vectors -> 0;
    # block 2: one zero key (-> 0 for it, not counted for the others)
    K = np.zeros((1, 1, 3 * b, d))
    K[0, 0, 0:b] = v
    for a in range(b):
        K[0, 0, b + a, a] = 1.0 + a
    K[0, 0, 2 * b:3 * b] = rng.standard_normal((b, d))
    K[0, 0, 2 * b + 1] = 0.0
    Rr = _lrs(K, b, 3, d)[0, 0]
    np.testing.assert_allclose(Rr[0:b], 1.0, atol=1e-15)
    np.testing.assert_array_equal(Rr[b:2 * b], 0.0)
    assert Rr[2 * b + 1] == 0.0
    ref = bf.lrs_sklearn(_as_stored(K[0, 0]), b)
    np.testing.assert_allclose(Rr, ref, atol=1e-14)


def test_lrs_antipodal_pair_b2():
    d, b = 4, 2
    k = np.array([1.0, -2.0, 0.5, 3.0])
    K = np.zeros((1, 1, 2 * b, d))
    K[0, 0, 0], K[0, 0, 1] = k, -k
    K[0, 0, 2], K[0, 0, 3] = k, 2.5 * k
    Rr = _lrs(K, b, 2, d)[0, 0]
    np.testing.assert_allclose(Rr, [-1.0, -1.0, 1.0, 1.0], atol=1e-15)


def test_lrs_matches_sklearn_and_is_block_local_and_scale_free():
    d, b, n_max = 8, 4, 6
    rng = np.random.default_rng(14)
    K = rng.standard_normal((2, 2, n_max * b, d))
    Rr = _lrs(_as_stored(K), b, n_max, d)
    for r in range(2):
        for h in range(2):
            np.testing.assert_allclose(Rr[r, h], bf.lrs_sklearn(_as_stored(K[r, h]), b),
                                       atol=1e-14)
    # changing every key outside block 2 leaves block 2's scores unchanged
    K2 = rng.standard_normal(K.shape)
    K2[:, :, 2 * b:3 * b] = K[:, :, 2 * b:3 * b]
    R2 = _lrs(K2, b, n_max, d)
    np.testing.assert_array_equal(R2[:, :, 2 * b:3 * b], Rr[:, :, 2 * b:3 * b])
    # positive rescaling of single keys leaves every cosine unchanged (powers
    # of two, so the float32 pool holds the scaled keys exactly)
    K3 = _as_stored(K) * np.exp2(rng.integers(-4, 5, size=K.shape[:3]))[..., None]
    np.testing.assert_allclose(_lrs(K3, b, n_max, d), Rr, atol=1e-13)
    # the pages' cost claim: N*b*(b-1) ordered pairs instead of (N*b)*(N*b-1)
    N = n_max
    assert N * b * (b - 1) < (N * b) * (N * b - 1)


# ---------------------------------------------------------------- all-pairs redundancy

def test_redundancy_all_closed_form_and_library():
    """Mean cosine with all other slots equals (u_j . sum_c u_c - 1)/(T-1)
    with u the unit keys (a different formula), and sklearn's cosine matrix."""
    from sklearn.metrics.pairwise import cosine_similarity
    rng = np.random.default_rng(41)
    R, H, d, b, n = 2, 2, 8, 4, 5
    T = n * b
    tables, kpool, _, K, _ = _tiny_case(rng, R=R, H=H, d=d, b=b, n_max=n, w=1, pool=16)
    got = oracle.redundancy_all(kpool, tables)
    for r in range(R):
        for h in range(H):
            Kl = bf.logical_rows(kpool, tables[r], h, T)
            U = Kl / np.linalg.norm(Kl, axis=1, keepdims=True)
            closed = (U @ U.sum(axis=0) - 1.0) / (T - 1)
            np.testing.assert_allclose(got[r, h], closed, atol=1e-13)
            C = cosine_similarity(Kl)
            np.testing.assert_allclose(got[r, h], (C.sum(axis=1) - 1.0) / (T - 1), atol=1e-13)


def test_redundancy_all_special_cases_and_block_case():
    d, b = 6, 4
    # identical keys -> 1; antipodal halves -> mean of +1 and -1 terms; a
    # zero key contributes 0 to the others and has 0 itself
    k = np.arange(1.0, d + 1.0)
    same = np.broadcast_to(k, (1, 1, 2 * b, d)).copy()
    tab = np.array([[3, 1]], dtype=np.int32)
    got = oracle.redundancy_all(synth.pool_from_logical(same, tab, 4, "f32"), tab)
    np.testing.assert_allclose(got, 1.0, atol=1e-15)
    anti = same.copy()
    anti[0, 0, b:] *= -1.0
    got = oracle.redundancy_all(synth.pool_from_logical(anti, tab, 4, "f32"), tab)
    np.testing.assert_allclose(got, ((b - 1) - b) / (2 * b - 1), atol=1e-15)
    zero = same.copy()
    zero[0, 0, 0] = 0.0
    got = oracle.redundancy_all(synth.pool_from_logical(zero, tab, 4, "f32"), tab)
    assert got[0, 0, 0] == 0.0
    np.testing.assert_allclose(got[0, 0, 1:], (2 * b - 2) / (2 * b - 1), atol=1e-15)
    # one block: the all-pairs score is the Lightning Redundancy Score
    rng = np.random.default_rng(42)
    tables, kpool, q, _, _ = _tiny_case(rng, R=1, H=2, Hq=2, d=8, b=4, n_max=1, w=1, pool=6)
    _, lrs, _ = oracle.scores(kpool, q, tables, num_kv_heads=2, num_q_heads=2, head_dim=8,
                              block_size=4, window=1)
    np.testing.assert_allclose(oracle.redundancy_all(kpool, tables), lrs, atol=1e-14)


# ---------------------------------------------------------------- selection

@pytest.mark.parametrize("seed", range(6))
def test_select_matches_exhaustive_search(seed):
    rng = np.random.default_rng(100 + seed)
    T, w = 12, 2
    C = T - w
    s = np.full(T, np.nan)
    s[:C] = rng.integers(0, 4, size=C).astype(np.float64)   # many exact ties
    for k_sel in (1, 3, 6, 9):
        kept = oracle.select(s[None], w, k_sel)[0]
        want = bf.select_exhaustive(list(s[:C].astype(int)), k_sel)
        assert kept.tolist() == want + list(range(C, T))


def test_select_dominance_and_window_on_random_scores():
    rng = np.random.default_rng(15)
    T, w, k_sel = 300, 16, 250
    C = T - w
    s = np.full((3, T), np.nan)
    s[:, :C] = rng.random((3, C))
    s[1, :C] = np.round(s[1, :C] * 20)   # heavy ties
    kept = oracle.select(s, w, k_sel)
    for u in range(3):
        kp = kept[u]
        assert np.all(np.diff(kp) > 0)
        assert set(range(C, T)) <= set(kp.tolist())
        sel = set(kp.tolist()) - set(range(C, T))
        ev = set(range(C)) - sel
        assert len(sel) == k_sel
        for k in sel:
            for e in ev:
                assert s[u, k] > s[u, e] or (s[u, k] == s[u, e] and k < e)


def test_select_exact_tie_evicts_highest_candidates():
    """q = 0 and orthogonal keys inside every block: every candidate gets the
    bit-identical score, so the tie rule evicts the E highest candidate slots."""
    d, b, n_max, w = 8, 4, 5, 3
    T = n_max * b
    C = T - w
    K = np.zeros((1, 1, T, d))
    for j in range(T):
        K[0, 0, j, j % b] = 1.0 + (j % 3)
    tables = np.arange(n_max, dtype=np.int32)[None]
    kpool = synth.pool_from_logical(K, tables, n_max, "f32")
    q = np.zeros((1, w, 1, d), dtype=np.float32)
    _, Rr, s = oracle.scores(kpool, q, tables, num_kv_heads=1, num_q_heads=1, head_dim=d,
                             block_size=b, n_max=n_max, window=w)
    assert np.all(Rr == 0.0)
    assert np.all(s[0, 0, :C] == s[0, 0, 0])
    k_sel = (n_max - 1) * b - w
    kept = oracle.select(s, w, k_sel)[0, 0]
    E = C - k_sel
    assert kept.tolist() == list(range(C - E)) + list(range(C, T))


# ---------------------------------------------------------------- compaction

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compaction_moves_exact_bytes_in_order(dtype):
    c = synth.make_case("pin", 21, num_reqs=3, num_layers=1, num_kv_heads=2, num_q_heads=4,
                        head_dim=8, block_size=4, n_max=6, window=2, num_blocks=40, dtype=dtype)
    res = oracle.compress(c)
    b, n_max = 4, 6
    k_keep = (n_max - 1) * b
    used = set(res.plan.dst.reshape(-1).tolist())
    for r in range(3):
        for h in range(2):
            kept = res.kept[0][r, h]
            before = bf.logical_rows(c.k_pool[0], res.plan.src[r], h, n_max * b)
            after = bf.logical_rows(res.k_pool[0], res.plan.tables[r], h, k_keep)
            np.testing.assert_array_equal(after, before[kept])
            vb = bf.logical_rows(c.v_pool[0], res.plan.src[r], h, n_max * b)
            va = bf.logical_rows(res.v_pool[0], res.plan.tables[r], h, k_keep)
            np.testing.assert_array_equal(va, vb[kept])
    # blocks that are not compaction targets are bit-for-bit untouched
    others = [i for i in range(40) if i not in used]
    np.testing.assert_array_equal(res.k_pool[0][others].view(np.uint8),
                                  c.k_pool[0][others].view(np.uint8))


# ---------------------------------------------------------------- planning

def test_plan_private_requests_compact_in_place():
    c = synth.case_tiny()
    p = oracle.plan(c.refcounts, c.tables, c.n_max)
    assert p.status == oracle.OK
    np.testing.assert_array_equal(p.tables, c.tables)
    np.testing.assert_array_equal(p.dst, c.tables[:, :-1])
    np.testing.assert_array_equal(p.refcounts, c.refcounts)
    assert p.freed.size == 0


def test_plan_shared_prefix_retargets_and_frees():
    R, n_max, P, pool = 4, 6, 2, 40
    c = synth.make_case("pfx", 22, num_reqs=R, num_layers=1, num_kv_heads=1, num_q_heads=1,
                        head_dim=8, block_size=4, n_max=n_max, window=2, num_blocks=pool,
                        dtype="f32", shared_prefix_blocks=P)
    prefix = c.tables[0, :P].tolist()
    assert all(c.refcounts[x] == R for x in prefix)
    free0 = sorted(np.flatnonzero(c.refcounts == 0).tolist())
    p = oracle.plan(c.refcounts, c.tables, n_max)
    assert p.status == oracle.OK
    # every request re-targets the shared blocks to the smallest free ids, in order
    assert p.dst[:, :P].reshape(-1).tolist() == free0[: R * P]
    np.testing.assert_array_equal(p.dst[:, P:], c.tables[:, P:n_max - 1])
    assert sorted(p.freed.tolist()) == sorted(prefix)
    assert all(p.refcounts[x] == 0 for x in prefix)
    # conservation: every count equals the number of table references
    want = np.zeros(pool, dtype=np.int32)
    np.add.at(want, p.tables.reshape(-1), 1)
    np.testing.assert_array_equal(p.refcounts, want)
    assert all(x not in p.tables for x in p.freed)
    assert (p.tables.shape[1] == n_max)


def test_plan_shared_reserved_block_is_replaced():
    tables = np.array([[3, 4, 5], [6, 7, 5]], dtype=np.int32)
    rc = np.zeros(10, dtype=np.int32)
    np.add.at(rc, tables.reshape(-1), 1)
    p = oracle.plan(rc, tables, 3)
    assert p.status == oracle.OK
    assert p.tables.tolist() == [[3, 4, 0], [6, 7, 1]]
    assert p.dst.tolist() == [[3, 4], [6, 7]]
    assert p.freed.tolist() == [5]


def test_plan_keeps_shared_blocks_below_the_first_eviction():
    """With the first evicted slot known, a shared block wholly below it
    stays in the table, still shared; one reaching past it is re-targeted."""
    b = 4
    tables = np.array([[3, 4, 5, 6], [3, 4, 7, 8]], dtype=np.int32)   # 3, 4 shared
    rc = np.zeros(16, dtype=np.int32)
    np.add.at(rc, tables.reshape(-1), 1)
    # request 0: first eviction at slot 8 -> blocks 0, 1 (slots 0..7) stay;
    # request 1: first eviction at slot 7 -> block 0 stays, block 1 (4..7) moves
    p = oracle.plan(rc, tables, 4, first_evict=np.array([8, 7]), block_size=b)
    assert p.status == oracle.OK
    assert p.tables.tolist() == [[3, 4, 5, 6], [3, 0, 7, 8]]
    assert p.dst.tolist() == [[3, 4, 5], [3, 0, 7]]
    assert p.refcounts[3] == 2 and p.refcounts[4] == 1 and p.refcounts[0] == 1
    assert p.freed.size == 0
    # without it every shared position is re-targeted
    q = oracle.plan(rc, tables, 4)
    assert q.tables.tolist() == [[0, 1, 5, 6], [2, 9, 7, 8]]
    assert sorted(q.freed.tolist()) == [3, 4]


def test_first_evicted_takes_the_lowest_slot_over_layers_and_heads():
    """Hand-built kept lists (T = 16, w = 2, so C = 14 candidates; 12 kept,
    4 evicted per head) whose first evictions differ by layer and head.
    Request 0: layer 0 first evicts 5 (head 0) and 3 (head 1), layer 1 4 and
    7 -> 3.  Request 1: 10, 9 | 10, 6 -> 6, the minimum sitting in the other
    layer and head.  Request 2: every head evicts 10..13 -> 10.  Evicted
    sets that are not runs (head 1 of request 0, layer 0: {3, 9, 10, 11})
    make a slip to the last eviction, or to the first kept slot, fail."""
    T, w = 16, 2
    evicted = {  # (layer, request, head) -> evicted candidate slots
        (0, 0, 0): {5, 6, 7, 8}, (0, 0, 1): {3, 9, 10, 11},
        (1, 0, 0): {4, 5, 12, 13}, (1, 0, 1): {7, 8, 9, 10},
        (0, 1, 0): {10, 11, 12, 13}, (0, 1, 1): {9, 11, 12, 13},
        (1, 1, 0): {10, 11, 12, 13}, (1, 1, 1): {6, 13, 12, 8},
        (0, 2, 0): {10, 11, 12, 13}, (0, 2, 1): {10, 11, 12, 13},
        (1, 2, 0): {10, 11, 12, 13}, (1, 2, 1): {10, 11, 12, 13},
    }
    kept = []
    for layer in range(2):
        k = np.zeros((3, 2, T - 4), dtype=np.int32)
        for r in range(3):
            for h in range(2):
                ev = evicted[(layer, r, h)]
                assert len(ev) == 4 and max(ev) < T - w
                k[r, h] = sorted(set(range(T)) - ev)
        kept.append(k)
    np.testing.assert_array_equal(oracle.first_evicted(kept, T, w), [3, 6, 10])
    # one layer alone: request 0 -> min(5, 3), request 1 -> min(10, 9)
    np.testing.assert_array_equal(oracle.first_evicted(kept[:1], T, w), [3, 9, 10])
    # the other alone: request 0 -> min(4, 7), request 1 -> min(10, 6)
    np.testing.assert_array_equal(oracle.first_evicted(kept[1:], T, w), [4, 6, 10])


def test_keep_prefix_compression_leaves_the_shared_prefix_in_place():
    """Exact ties (zero queries, axis-aligned keys): the evicted candidates
    are the highest slots, far past a 2-block shared prefix, which then stays
    shared with unchanged bytes while the rest compacts as usual."""
    R, H, d, b, n_max, w, P = 3, 2, 16, 4, 6, 2, 2
    c = synth.make_case("kp", 43, num_reqs=R, num_layers=2, num_kv_heads=H, num_q_heads=H,
                        head_dim=d, block_size=b, n_max=n_max, window=w, num_blocks=40,
                        dtype="f32", shared_prefix_blocks=P)
    T = n_max * b
    K = np.zeros((R, H, T, d))
    for j in range(T):
        K[:, :, j, j % b] = 1.0 + (j % 3)
    for l in range(2):
        c.k_pool[l] = synth.pool_from_logical(K, c.tables, 40, "f32")
        c.window_q[l] = np.zeros_like(c.window_q[l])
    res = oracle.compress(c, keep_prefix=True)
    prefix = c.tables[0, :P]
    assert np.all(res.plan.tables[:, :P] == prefix)
    assert all(res.plan.refcounts[x] == R for x in prefix) and res.plan.freed.size == 0
    C, E = T - w, b
    for l in range(2):
        want = list(range(C - E)) + list(range(C, T))
        assert np.all(res.kept[l] == np.array(want))
        np.testing.assert_array_equal(res.k_pool[l][prefix], c.k_pool[l][prefix])
    # the plain compression re-targets the same prefix into new blocks
    plain = oracle.compress(c)
    assert not np.any(np.isin(plain.plan.tables[:, :P], prefix))


def test_plan_over_cap_releases_the_surplus():
    """A request holding n_src > n_max blocks keeps its first n_max-1 blocks
    as targets and block n_max-1 as the reserved one; blocks n_max.. are
    released (freed when this was their last reference)."""
    # request 0: private blocks; request 1 shares a surplus block with request 2
    tables = np.array([[3, 4, 5, 6, 7], [8, 9, 10, 11, 12], [13, 14, 15, 16, 12]], dtype=np.int32)
    rc = np.zeros(20, dtype=np.int32)
    np.add.at(rc, tables.reshape(-1), 1)
    p = oracle.plan(rc, tables, 3)
    assert p.status == oracle.OK
    assert p.tables.tolist() == [[3, 4, 5, -1, -1], [8, 9, 10, -1, -1], [13, 14, 15, -1, -1]]
    assert p.dst.tolist() == [[3, 4], [8, 9], [13, 14]]
    np.testing.assert_array_equal(p.src, tables)
    # 6, 7, 11, 16 were private: freed; 12 was held twice: freed by request 2
    assert sorted(p.freed.tolist()) == [6, 7, 11, 12, 16]
    want = np.zeros(20, dtype=np.int32)
    np.add.at(want, p.tables[p.tables >= 0], 1)
    np.testing.assert_array_equal(p.refcounts, want)
    # a surplus block also held by a request outside the call stays allocated
    rc_ext = rc.copy()
    rc_ext[7] += 1
    p2 = oracle.plan(rc_ext, tables, 3)
    assert 7 not in p2.freed.tolist() and p2.refcounts[7] == 1


def test_over_cap_case_end_to_end_invariants():
    """n_src = n_max + 2: E = 3b evictions per head, the window kept, the
    survivors in order in the first n_max-1 blocks, the surplus freed."""
    c = synth.make_case("over", 28, num_reqs=2, num_layers=1, num_kv_heads=2, num_q_heads=4,
                        head_dim=16, block_size=4, n_max=5, window=3, num_blocks=24, dtype="f32",
                        n_src=7)
    b, n_max, n_src, w = 4, 5, 7, 3
    T, k_keep = n_src * b, (n_max - 1) * b
    res = oracle.compress(c)
    kept = res.kept[0]
    assert kept.shape == (2, 2, k_keep)
    for r in range(2):
        assert sorted(res.plan.freed.tolist()) == sorted(c.tables[:, n_max:].reshape(-1).tolist())
        for h in range(2):
            k = kept[r, h]
            assert np.all(np.diff(k) > 0) and k[-w:].tolist() == list(range(T - w, T))
            # the evicted candidates never beat a kept one
            ev = sorted(set(range(T - w)) - set(k.tolist()))
            assert len(ev) == T - k_keep
            s = res.s[0][r, h]
            assert max(s[e] for e in ev) <= min(s[j] for j in k[:-w])
            # compacted rows are the kept source rows, read through the old table
            for slot in range(k_keep):
                j = k[slot]
                want = c.k_pool[0][c.tables[r, j // b], h, j % b]
                got = res.k_pool[0][res.plan.tables[r, slot // b], h, slot % b]
                np.testing.assert_array_equal(got, want)


def test_plan_all_or_nothing_errors():
    tables = np.array([[3, 4, 5], [6, 7, 5]], dtype=np.int32)
    rc = np.zeros(8, dtype=np.int32)
    np.add.at(rc, tables.reshape(-1), 1)
    rc_small = rc.copy()
    # free blocks 0,1,2: enough for two new reserved blocks
    assert oracle.plan(rc, tables, 3).status == oracle.OK
    # only one free block left -> no change, NO_BLOCKS
    rc_small[[0, 1]] = 1
    p = oracle.plan(rc_small, tables, 3)
    assert p.status == oracle.NO_BLOCKS
    bad = [
        np.array([[3, 3, 5]], dtype=np.int32),   # duplicate inside a table
        np.array([[3, 4, 9]], dtype=np.int32),   # out of range
        np.array([[3, 4, 0]], dtype=np.int32),   # refcount 0
    ]
    for t in bad:
        assert oracle.plan(rc, t, 3).status == oracle.INVALID
    # more appearances than references
    rc1 = rc.copy()
    rc1[5] = 1
    assert oracle.plan(rc1, tables, 3).status == oracle.INVALID


# ---------------------------------------------------------------- decode

def test_decode_equal_keys_gives_mean_of_values():
    rng = np.random.default_rng(23)
    H, Hq, d, b, n = 2, 4, 8, 4, 13
    K = np.broadcast_to(rng.standard_normal(d), (1, H, 16, d)).copy()
    V = rng.standard_normal((1, H, 16, d))
    tables = np.array([[5, 1, 7, 2]], dtype=np.int32)
    kp = synth.pool_from_logical(K, tables, 8, "f32")
    vp = synth.pool_from_logical(V, tables, 8, "f32")
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    out = oracle.decode(kp, vp, q, tables, np.array([n], dtype=np.int32), num_q_heads=Hq)
    Vf = V.astype(np.float32).astype(np.float64)
    for hq in range(Hq):
        np.testing.assert_allclose(out[0, hq], Vf[0, hq // 2, :n].mean(axis=0), atol=1e-12)


def test_decode_dominant_logit_selects_one_value_row():
    rng = np.random.default_rng(24)
    H, Hq, d, b = 1, 2, 8, 4
    K = rng.standard_normal((1, H, 12, d)) * 0.01
    q = rng.standard_normal((1, Hq, d))
    K[0, 0, 6] = 50.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    V = rng.standard_normal((1, H, 12, d))
    tables = np.array([[2, 0, 1]], dtype=np.int32)
    kp = synth.pool_from_logical(K, tables, 3, "f32")
    vp = synth.pool_from_logical(V, tables, 3, "f32")
    out = oracle.decode(kp, vp, q.astype(np.float32), tables, np.array([12], dtype=np.int32),
                        num_q_heads=Hq, scale=1.0)
    np.testing.assert_allclose(out[0, 0], V.astype(np.float32)[0, 0, 6], atol=1e-9)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_lse_matches_scipy_logsumexp(dtype):
    from scipy.special import logsumexp
    c = synth.make_case("lse", 26, num_reqs=3, num_layers=1, num_kv_heads=2, num_q_heads=6,
                        head_dim=16, block_size=4, n_max=5, window=2, num_blocks=20, dtype=dtype)
    seq = np.array([20, 13, 0], dtype=np.int32)
    lse = oracle.decode_lse(c.k_pool[0], c.q_new[0], c.tables, seq, num_q_heads=6)
    qf = c.q_new[0] if dtype == "f32" else synth.bf16_bits_to_f32(c.q_new[0])
    for r in range(2):
        for hq in range(6):
            Kl = bf.logical_rows(c.k_pool[0], c.tables[r], hq // 3, int(seq[r]))
            want = logsumexp(Kl @ qf[r, hq].astype(np.float64) / 4.0)
            assert abs(lse[r, hq] - want) <= 1e-12 * max(1.0, abs(want))
    assert np.all(np.isneginf(lse[2]))  # empty request


def test_decode_lse_equal_keys_closed_form():
    rng = np.random.default_rng(27)
    H, Hq, d, n = 1, 2, 8, 11
    k = rng.standard_normal(d)
    K = np.broadcast_to(k, (1, H, 12, d)).copy()
    tables = np.array([[2, 0, 1]], dtype=np.int32)
    kp = synth.pool_from_logical(K, tables, 3, "f32")
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    lse = oracle.decode_lse(kp, q, tables, np.array([n], dtype=np.int32), num_q_heads=Hq,
                            scale=0.5)
    kf = k.astype(np.float32).astype(np.float64)
    for hq in range(Hq):
        want = np.log(n) + 0.5 * float(q[0, hq].astype(np.float64) @ kf)
        assert abs(lse[0, hq] - want) <= 1e-12 * max(1.0, abs(want))


@pytest.mark.parametrize("G,w", [(1, 2), (4, 3)])
def test_window_lse_normalises_the_importance_rows(G, w):
    """The decode log-sum-exp of window query i over slots 0..T-w+i is the
    normaliser of importance row i: recomputing A from it (dense logits in
    NumPy) gives the oracle's A."""
    rng = np.random.default_rng(31 + G)
    H, d, b, n_max = 2, 8, 4, 6
    T = n_max * b
    tables, kpool, q, K, Q = _tiny_case(rng, H=H, Hq=H * G, d=d, b=b, n_max=n_max, w=w)
    A, _, _ = oracle.scores(kpool, q, tables, num_kv_heads=H, num_q_heads=H * G, head_dim=d,
                            block_size=b, n_max=n_max, window=w)
    lse = oracle.window_lse(kpool, q, tables, n_max=n_max, window=w, num_q_heads=H * G)
    Qf = q.astype(np.float64)
    for r in range(2):
        for h in range(H):
            Kl = bf.logical_rows(kpool, tables[r], h, T)
            acc = np.zeros(T)
            for i in range(w):
                for g in range(G):
                    x = Kl[: T - w + i + 1] @ Qf[r, i, h * G + g] / np.sqrt(d)
                    acc[: T - w + i + 1] += np.exp(x - lse[r, i, h * G + g])
            np.testing.assert_allclose(A[r, h], acc / (G * w), rtol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_matches_torch_sdpa(dtype):
    c = synth.make_case("dec", 25, num_reqs=3, num_layers=1, num_kv_heads=2, num_q_heads=6,
                        head_dim=16, block_size=4, n_max=5, window=2, num_blocks=20, dtype=dtype)
    seq = np.array([20, 13, 1], dtype=np.int32)
    out = oracle.decode(c.k_pool[0], c.v_pool[0], c.q_new[0], c.tables, seq, num_q_heads=6)
    qf = c.q_new[0] if dtype == "f32" else synth.bf16_bits_to_f32(c.q_new[0])
    for r in range(3):
        for hq in range(6):
            h = hq // 3
            Kl = bf.logical_rows(c.k_pool[0], c.tables[r], h, int(seq[r]))
            Vl = bf.logical_rows(c.v_pool[0], c.tables[r], h, int(seq[r]))
            ref = bf.decode_sdpa(Kl, Vl, qf[r, hq].astype(np.float64), 1.0 / 4.0)
            np.testing.assert_allclose(out[r, hq], ref, atol=1e-12)


def test_append_writes_one_row_per_head():
    c = synth.case_tiny()
    kp, vp = c.k_pool[0].copy(), c.v_pool[0].copy()
    slot = np.array([int(c.tables[0, 7]) * 16 + 0], dtype=np.int32)
    oracle.append(kp, vp, c.k_new[0], c.v_new[0], slot)
    blk = int(c.tables[0, 7])
    np.testing.assert_array_equal(kp[blk, :, 0], c.k_new[0][0])
    np.testing.assert_array_equal(vp[blk, :, 0], c.v_new[0][0])
    mask = np.ones(kp.shape[:3], dtype=bool)
    mask[blk, :, 0] = False
    np.testing.assert_array_equal(kp[mask].view(np.uint32), c.k_pool[0][mask].view(np.uint32))


# ---------------------------------------------------------------- end to end invariants

def test_tiny_case_end_to_end_invariants():
    c = synth.case_tiny()
    res = oracle.compress(c)
    b, n_max, w = 16, 8, 8
    T, k_keep = n_max * b, (n_max - 1) * b
    kept = res.kept[0]
    assert kept.shape == (1, 2, k_keep)
    for h in range(2):
        assert kept[0, h, -w:].tolist() == list(range(T - w, T))
    assert res.plan.tables.shape == (1, n_max)
    # the reserved block stays and the pending token lands at slot k_keep
    assert res.plan.tables[0, -1] == c.tables[0, -1]
    kp, vp = res.k_pool[0].copy(), res.v_pool[0].copy()
    slot = np.array([res.plan.tables[0, k_keep // b] * b + k_keep % b], dtype=np.int32)
    oracle.append(kp, vp, c.k_new[0], c.v_new[0], slot)
    out = oracle.decode(kp, vp, c.q_new[0], res.plan.tables, np.array([k_keep + 1], dtype=np.int32),
                        num_q_heads=4)
    assert np.isfinite(out).all()


def test_bf16_inputs_are_widened_exactly():
    """Scores from a bf16 pool equal scores from the same values stored as f32."""
    rng = np.random.default_rng(26)
    tables, kpool16, q16, _, _ = _tiny_case(rng, dtype="bf16")
    kpool32 = synth.bf16_bits_to_f32(kpool16)
    q32 = synth.bf16_bits_to_f32(q16)
    kw = dict(num_kv_heads=2, num_q_heads=4, head_dim=8, block_size=4, n_max=5, window=3)
    a = oracle.scores(kpool16, q16, tables, **kw)
    b = oracle.scores(kpool32, q32, tables, **kw)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------------- requests holding different counts

def test_plan_with_per_request_block_counts_by_hand():
    """n_max = 3.  Request 0 holds 3 blocks [2, 3, 4]; request 1 holds 5
    blocks [5, 6, 7, 8, 9], block 6 also held by someone outside the call.
    Request 0 compacts in place.  Request 1: block 5 in place; block 6 is
    shared, so it gets the smallest free id, 0, and drops to count 1 (not
    freed); block 7 is its reserved block; blocks 8 and 9 are surplus, count
    0: freed.  Rows stay padded with -1 past each request's blocks."""
    tables = np.array([[2, 3, 4, -1, -1], [5, 6, 7, 8, 9]], dtype=np.int32)
    rc = np.zeros(16, dtype=np.int32)
    np.add.at(rc, tables[tables >= 0], 1)
    rc[6] += 1
    p = oracle.plan(rc, tables, 3, n_blocks=np.array([3, 5]))
    assert p.status == oracle.OK
    assert p.tables.tolist() == [[2, 3, 4, -1, -1], [5, 0, 7, -1, -1]]
    assert p.dst.tolist() == [[2, 3], [5, 0]]
    assert sorted(p.freed.tolist()) == [8, 9]
    assert p.refcounts[0] == 1 and p.refcounts[6] == 1 and p.refcounts[8] == 0
    # a row not padded with -1 past its count, or a count outside [n_max, n_src]
    bad = tables.copy()
    bad[0, 3] = 11
    assert oracle.plan(rc, bad, 3, n_blocks=np.array([3, 5])).status == oracle.INVALID
    assert oracle.plan(rc, tables, 3, n_blocks=np.array([2, 5])).status == oracle.INVALID
    assert oracle.plan(rc, tables, 3, n_blocks=np.array([3, 6])).status == oracle.INVALID


def test_ragged_compression_is_each_request_on_its_own():
    """Requests holding 4, 6 and 5 blocks (n_max = 4) in one call, no block
    shared (so no allocation order is involved): the scores, survivors and
    compacted rows of each request equal those of the request compressed
    alone."""
    case = synth.make_case("ragged", 91, num_reqs=3, num_layers=2, num_kv_heads=2, num_q_heads=4,
                           head_dim=16, block_size=4, n_max=4, window=3, num_blocks=24,
                           dtype="f32", n_src=[4, 6, 5])
    assert case.num_blocks.tolist() == [4, 6, 5] and case.tables.shape == (3, 6)
    assert np.all(case.tables[0, 4:] == -1) and np.all(case.tables[2, 5:] == -1)
    res = oracle.compress(case)
    b = 4
    for r, n in enumerate(case.num_blocks.tolist()):
        alone = synth.CompressCase("alone", 0, case.geom, case.n_max, case.window,
                                   np.ascontiguousarray(case.tables[r:r + 1, :n]),
                                   case.refcounts, case.k_pool, case.v_pool,
                                   [q[r:r + 1] for q in case.window_q], [], [], [])
        one = oracle.compress(alone)
        assert one.plan.tables[0, :4].tolist() == res.plan.tables[r, :4].tolist()
        for l in range(2):
            np.testing.assert_array_equal(res.A[l][r, :, :n * b], one.A[l][0])
            np.testing.assert_array_equal(res.s[l][r, :, :n * b], one.s[l][0])
            assert np.isnan(res.A[l][r, :, n * b:]).all()
            np.testing.assert_array_equal(res.kept[l][r], one.kept[l][0])
            for a, c in ((res.k_pool[l], one.k_pool[l]), (res.v_pool[l], one.v_pool[l])):
                tgt = res.plan.dst[r]
                np.testing.assert_array_equal(a[tgt], c[tgt])
    # surplus blocks released: 2 + 1 of them
    assert sorted(res.plan.freed.tolist()) == sorted(case.tables[1, 4:6].tolist()
                                                    + case.tables[2, 4:5].tolist())
