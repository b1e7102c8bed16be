"""Host-side checks of the C ABI (no GPU work): symbols, block pool,
planner parity with the oracle, and argument validation."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import compressed_paged_kv_amd as zp
import oracle
import synth
from compressed_paged_kv_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*[\w\s\*]+?\b(zp_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert "zp_compress" in names and "zp_paged_decode" in names and "zp_block_alloc" in names
    lib = zp.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (zp_\w+)", out))
    assert set(names) <= exported
    assert zp.lib().zp_version() == 2


def test_library_links_no_oracle():
    out = subprocess.run(["nm", "-D", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "zpo_" not in out
    deps = subprocess.run(["ldd", B.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps


# ------------------------------------------------------------------ block pool

def test_pool_alloc_smallest_first_and_all_or_nothing():
    p = zp.BlockPool(8, manual_fence=True)
    assert p.alloc(3).tolist() == [0, 1, 2]
    p.release([1])
    assert p.alloc(2).tolist() == [1, 3]
    assert p.num_free() == 4
    with pytest.raises(zp.ZpError) as e:
        p.alloc(5)
    assert e.value.status == zp.ZP_ERR_NO_BLOCKS
    assert p.num_free() == 4
    assert [p.refcount(i) for i in range(8)] == [1, 1, 1, 1, 0, 0, 0, 0]


def test_pool_share_release_and_errors():
    p = zp.BlockPool(6, manual_fence=True)
    ids = p.alloc(2)
    p.share([ids[0], ids[0]])
    assert p.refcount(ids[0]) == 3
    assert p.release([ids[0]]).tolist() == []
    assert p.release([ids[0], ids[0], ids[1]]).tolist() == [ids[0], ids[1]]
    assert p.num_free() == 6
    for bad in ([7], [-1]):
        with pytest.raises(zp.ZpError) as e:
            p.share(bad)
        assert e.value.status == zp.ZP_ERR_INVALID
    with pytest.raises(zp.ZpError):
        p.share([2])                  # not allocated
    x = p.alloc(1)
    with pytest.raises(zp.ZpError):
        p.release([x[0], x[0]])       # more releases than references
    assert p.refcount(int(x[0])) == 1
    assert p.refcount(99) == -1


def test_pool_from_refcounts_roundtrip():
    rc = np.array([0, 2, 1, 0, 5, 1], dtype=np.int32)
    p = zp.BlockPool.from_refcounts(rc, manual_fence=True)
    np.testing.assert_array_equal(p.refcounts(), rc)
    assert p.num_free() == 2


# ------------------------------------------------------------------ planner

def _scenario(seed):
    """Random tables with shared blocks and external holders; every third
    seed the requests hold more than n_max blocks (a cache past the cap)."""
    rng = np.random.default_rng(seed)
    pool = int(rng.integers(40, 90))
    n_max = int(rng.integers(2, 7))
    n_src = n_max + (int(rng.integers(1, 4)) if seed % 3 == 2 else 0)
    R = int(rng.integers(1, 6))
    ids = rng.permutation(pool)
    tables = ids[: R * n_src].reshape(R, n_src).astype(np.int32)
    # share some blocks between requests (prefix-like and random)
    if R > 1 and rng.random() < 0.8:
        P = int(rng.integers(1, n_max + 1))
        tables[:, :P] = tables[0, :P]
    for _ in range(int(rng.integers(0, 3))):
        r1, r2 = rng.integers(0, R, size=2)
        n1, n2 = rng.integers(0, n_src, size=2)
        if r1 != r2 and tables[r2, n2] not in tables[r1]:
            tables[r1, n1] = tables[r2, n2]
    rc = np.zeros(pool, dtype=np.int32)
    np.add.at(rc, tables.reshape(-1), 1)
    # external holders (e.g. a prefix cache) on a few blocks
    for x in rng.choice(np.flatnonzero(rc > 0), size=2):
        rc[x] += int(rng.integers(0, 2))
    return tables, rc, n_max


@pytest.mark.parametrize("seed", range(40))
def test_planner_matches_oracle(seed):
    tables, rc, n_max = _scenario(seed)
    want = oracle.plan(rc, tables, n_max)
    pool = zp.BlockPool.from_refcounts(rc, manual_fence=True)
    tab = tables.copy()
    if want.status == oracle.NO_BLOCKS:
        with pytest.raises(zp.ZpError) as e:
            zp.compress_plan(pool, n_max, tab)
        assert e.value.status == zp.ZP_ERR_NO_BLOCKS
        np.testing.assert_array_equal(tab, tables)
        np.testing.assert_array_equal(pool.refcounts(), rc)
        return
    assert want.status == oracle.OK
    src, dst, freed = zp.compress_plan(pool, n_max, tab)
    np.testing.assert_array_equal(tab, want.tables)
    np.testing.assert_array_equal(src, want.src)
    np.testing.assert_array_equal(dst, want.dst[:, : n_max - 1])
    np.testing.assert_array_equal(freed, want.freed)
    np.testing.assert_array_equal(pool.refcounts(), want.refcounts)
    # freed blocks wait for the fence
    assert pool.num_pending() == freed.size
    before = pool.num_free()
    pool.fence()
    assert pool.num_pending() == 0
    assert pool.num_free() == before + freed.size
    # invariants: counts = table references + external holders; freed in no table
    ext = rc.copy()
    np.subtract.at(ext, tables.reshape(-1), 1)
    want_rc = ext.copy()
    np.add.at(want_rc, tab[tab >= 0], 1)
    np.testing.assert_array_equal(pool.refcounts(), want_rc)
    assert not set(freed.tolist()) & set(tab.reshape(-1).tolist())


def test_planner_invalid_inputs_change_nothing():
    tables = np.array([[3, 4, 5], [6, 7, 5]], dtype=np.int32)
    rc = np.zeros(10, dtype=np.int32)
    np.add.at(rc, tables.reshape(-1), 1)
    pool = zp.BlockPool.from_refcounts(rc, manual_fence=True)
    for bad in ([[3, 3, 5]], [[3, 4, 10]], [[3, 4, 0]], [[5, 4, 3], [5, 6, 7], [5, 1, 2]]):
        t = np.array(bad, dtype=np.int32)
        t0 = t.copy()
        with pytest.raises(zp.ZpError) as e:
            zp.compress_plan(pool, 3, t)
        assert e.value.status == zp.ZP_ERR_INVALID
        np.testing.assert_array_equal(t, t0)
        np.testing.assert_array_equal(pool.refcounts(), rc)
    with pytest.raises(zp.ZpError):
        zp.compress_plan(pool, 1, np.array([[3]], dtype=np.int32))


def test_planner_shared_prefix_case_conserves_refcounts():
    c = synth.make_case("pfx", 31, num_reqs=6, num_layers=1, num_kv_heads=1, num_q_heads=1,
                        head_dim=64, block_size=16, n_max=9, window=16, num_blocks=120,
                        dtype="f32", shared_prefix_blocks=4)
    pool = zp.BlockPool.from_refcounts(c.refcounts, manual_fence=True)
    tab = c.tables.copy()
    src, dst, freed = zp.compress_plan(pool, 9, tab)
    prefix = c.tables[0, :4]
    assert sorted(freed.tolist()) == sorted(prefix.tolist())
    assert all(pool.refcount(int(x)) == 0 for x in prefix)
    assert pool.num_pending() == 4
    total = sum(pool.refcount(i) for i in range(120))
    assert total == tab.size


# ------------------------------------------------------------------ validation

class _FakeTensor:
    """Host buffer posing as a device tensor (a cuda:0 device and a real torch
    dtype, so the binding's own checks pass) for calls that must fail in
    validation before touching any device memory."""

    def __init__(self, shape, dtype_name, nbytes=64):
        import torch
        self.shape = tuple(shape)
        self.dtype = getattr(torch, dtype_name.split(".")[-1])
        self.device = torch.device("cuda", 0)
        self._nbytes = max(nbytes, 64)
        self._buf = ctypes.create_string_buffer(self._nbytes + 256)
        self._ptr = (ctypes.addressof(self._buf) + 255) // 256 * 256

    def data_ptr(self):
        return self._ptr

    def is_contiguous(self):
        return True

    def numel(self):
        return self._nbytes

    def element_size(self):
        return 1


def _fake_cache(L=1, H=2, Hq=4, d=64, b=16, nb=16, dtype="torch.float32"):
    ks = [_FakeTensor((nb, H, b, d), dtype) for _ in range(L)]
    vs = [_FakeTensor((nb, H, b, d), dtype) for _ in range(L)]
    return zp.KVCache(ks, vs, Hq)


def _raw_compress(cache, pool, n_max, window, tables, wq, ws):
    """zp_compress through the C ABI alone (no binding checks): the library's
    own validation is what these tests pin."""
    lib = zp.lib()
    arr = (ctypes.c_void_p * cache.num_layers)(*[t.data_ptr() for t in wq])
    freed = np.zeros(max(tables.size, 1), dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    i32 = ctypes.POINTER(ctypes.c_int32)
    return lib.zp_compress(cache.ref, pool.handle, n_max, window, int(tables.shape[0]),
                           tables.ctypes.data_as(i32), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)),
                           ws.data_ptr(), ws.numel() * ws.element_size(),
                           freed.ctypes.data_as(i32), n.ctypes.data_as(i32), None, None)


def test_compress_rejects_bad_arguments_before_any_work():
    cache = _fake_cache()
    n_max = 8
    pool = zp.BlockPool(16)
    tables = np.arange(8, dtype=np.int32)[None].copy()
    pool.alloc(8)
    wq = [_FakeTensor((1, 8, 4, 64), "torch.float32")]
    ws = _FakeTensor((1,), "torch.uint8")
    for kwargs in (dict(window=0), dict(window=17), dict(n_max=1)):
        args = dict(n_max=n_max, window=8)
        args.update(kwargs)
        t = tables.copy()
        st = _raw_compress(cache, pool, args["n_max"], args["window"], t, wq, ws)
        assert st == zp.ZP_ERR_INVALID, (kwargs, zp.last_error())
        np.testing.assert_array_equal(t, tables)
    # workspace too small (the fake reports 64 bytes)
    with pytest.raises(zp.ZpError) as e:
        zp.compress(cache, pool, n_max, 8, tables.copy(), wq, ws, stream=0)
    assert e.value.status == zp.ZP_ERR_INVALID and "workspace" in str(e.value)
    assert [pool.refcount(i) for i in range(8)] == [1] * 8
    # manual-fence pools are for host planning only
    mpool = zp.BlockPool(16, manual_fence=True)
    with pytest.raises(zp.ZpError):
        zp.compress(cache, mpool, n_max, 8, tables.copy(), wq, ws, stream=0)


def test_compress_rejects_malformed_block_counts_before_any_work():
    """Requests holding different block counts: each count must lie in
    [n_max, n_src] and the rest of the row must be -1; otherwise the call
    fails in planning, with tables and refcounts unchanged."""
    cache = _fake_cache()
    n_max, n_src = 8, 11
    pool = zp.BlockPool(16)
    ids = pool.alloc(8 + 11 - 8)
    tables = np.full((2, n_src), -1, dtype=np.int32)
    tables[0, :8] = ids[:8]          # request 0 at the cap
    tables[1, :3] = ids[8:]          # request 1 needs 11 -> shares 8 of request 0's ids
    tables[1, 3:11] = ids[:8]
    for i in ids[:8]:
        pool.share([int(i)])
    rc0 = [pool.refcount(i) for i in range(16)]
    wq = [_FakeTensor((2, 8, 4, 64), "torch.float32")]
    need = zp.compress_workspace_bytes(cache, 2, n_max, 8, n_src=n_src)
    ws = _FakeTensor((need,), "torch.uint8", nbytes=need)
    bad = {
        "count below n_max": (np.array([7, 11], np.int32), tables),
        "count past n_src": (np.array([8, 12], np.int32), tables),
        "padding not -1": (np.array([8, 11], np.int32),
                           np.where(np.arange(n_src)[None] == 9, 3, tables).astype(np.int32)),
        "hole inside the count": (np.array([9, 11], np.int32), tables),
    }
    for what, (counts, tab) in bad.items():
        t = np.ascontiguousarray(tab).copy()
        with pytest.raises(zp.ZpError) as e:
            zp.compress(cache, pool, n_max, 8, t, wq, ws, stream=0, num_blocks=counts)
        assert e.value.status == zp.ZP_ERR_INVALID, (what, str(e.value))
        np.testing.assert_array_equal(t, tab)
        assert [pool.refcount(i) for i in range(16)] == rc0, what
    with pytest.raises(ValueError):       # the binding checks the shape itself
        zp.compress(cache, pool, n_max, 8, tables.copy(), wq, ws, stream=0,
                    num_blocks=np.array([8], np.int32))


def test_compress_rejects_a_query_slot_store_without_slots():
    """window_slots needs window_store_slots >= 1 and 4-byte alignment; the
    binding needs the stores shaped [S*w][Hq][d] (and [S*w][Hq])."""
    import torch
    cache = _fake_cache()
    n_max = 8
    pool = zp.BlockPool(16)
    tables = np.arange(8, dtype=np.int32)[None].copy()
    pool.alloc(8)
    need = zp.compress_workspace_bytes(cache, 1, n_max, 8)
    ws = _FakeTensor((need,), "torch.uint8", nbytes=need)
    store = [_FakeTensor((3 * 8, 4, 64), "torch.float32")]
    slots = _FakeTensor((1,), "torch.int32")
    lib = zp.lib()
    wq = (ctypes.c_void_p * 1)(store[0].data_ptr())
    freed = np.zeros(8, dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    i32 = ctypes.POINTER(ctypes.c_int32)
    for ptr, count in ((slots.data_ptr(), 0), (slots.data_ptr() + 2, 3)):
        t = tables.copy()
        a = zp._binding._CompressArgs(8, n_max, 8, 1, t.ctypes.data_as(i32), None,
                                      ctypes.cast(wq, ctypes.POINTER(ctypes.c_void_p)), None,
                                      ws.data_ptr(), need, freed.ctypes.data_as(i32),
                                      n.ctypes.data_as(i32), None, None, 0, None, ptr, count)
        assert lib.zp_compress_ex(cache.ref, pool.handle, ctypes.byref(a)) == zp.ZP_ERR_INVALID
        assert "window_slots" in zp.last_error()
        np.testing.assert_array_equal(t, tables)
    with pytest.raises(ValueError):       # a dense [R][w][Hq][d] array is not a store
        zp.compress(cache, pool, n_max, 8, tables.copy(), [_FakeTensor((1, 8, 4, 64), "torch.float32")],
                    ws, stream=0, window_slots=slots)
    assert [pool.refcount(i) for i in range(8)] == [1] * 8


def test_binding_rejects_tensors_the_kernels_cannot_take():
    """The binding checks device, element type, contiguity and shape of every
    tensor before a pointer reaches the library (the C layer sees only
    addresses): a CPU tensor, an int64 table, a short window-query tensor or
    a strided view raise ValueError and nothing is called."""
    import torch
    cache = _fake_cache()
    pool = zp.BlockPool(16)
    tables = np.arange(8, dtype=np.int32)[None].copy()
    pool.alloc(8)
    ws = _FakeTensor((1,), "torch.uint8")
    good_wq = [_FakeTensor((1, 8, 4, 64), "torch.float32")]
    bad_wq = {
        "on the CPU": [torch.zeros((1, 8, 4, 64))],
        "dtype": [_FakeTensor((1, 8, 4, 64), "torch.bfloat16")],
        "shape": [_FakeTensor((1, 7, 4, 64), "torch.float32")],
    }
    for why, wq in bad_wq.items():
        with pytest.raises(ValueError):
            zp.compress(cache, pool, 8, 8, tables.copy(), wq, ws, stream=0)
    with pytest.raises(ValueError):
        zp.compress(cache, pool, 8, 8, tables.astype(np.int64), good_wq, ws, stream=0)
    with pytest.raises(ValueError):   # one entry per layer
        zp.compress(cache, pool, 8, 8, tables.copy(), good_wq * 2, ws, stream=0)
    assert [pool.refcount(i) for i in range(8)] == [1] * 8

    q = _FakeTensor((2, 4, 64), "torch.float32")
    tab = _FakeTensor((2, 8), "torch.int32")
    seq = _FakeTensor((2,), "torch.int32")
    out = _FakeTensor((2, 4, 64), "torch.float32")
    for args in ((torch.zeros((2, 4, 64)), tab, seq, out),                 # q on the CPU
                 (q, _FakeTensor((2, 8), "torch.int64"), seq, out),         # int64 table
                 (q, tab, _FakeTensor((3,), "torch.int32"), out),           # lengths of another batch
                 (q, tab, seq, _FakeTensor((2, 4, 64), "torch.bfloat16")),  # output not float32
                 (_FakeTensor((2, 4, 32), "torch.float32"), tab, seq, out)):
        with pytest.raises(ValueError):
            zp.paged_decode(cache, 0, *args, 0.125, None, stream=0)
    strided = torch.zeros((2, 4, 128))[..., ::2]
    with pytest.raises(ValueError):
        zp.paged_decode(cache, 0, strided, tab, seq, 0.125, out, None, stream=0)
    kv = _FakeTensor((2, 2, 64), "torch.float32")
    with pytest.raises(ValueError):
        zp.append_kv(cache, 0, kv, kv, _FakeTensor((2,), "torch.int64"), stream=0)
    with pytest.raises(ValueError):
        zp.append_kv(cache, 0, _FakeTensor((2, 4, 64), "torch.float32"), kv, seq, stream=0)
    with pytest.raises(ValueError):   # pools must live on a GPU
        zp.KVCache([torch.zeros((4, 2, 16, 64))], [torch.zeros((4, 2, 16, 64))], 4)


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("block_size", 8), ("num_q_heads", 6),
                                         ("num_q_heads", 32)])
def test_geometry_validation(field, value):
    cache = _fake_cache()
    setattr(cache.c, field, value)
    assert zp.lib().zp_compress_workspace_bytes(cache.ref, 1, 8, 8) == 0
    assert zp.last_error()


def test_workspace_sizes_grow_with_the_batch():
    cache = _fake_cache(L=2, H=8, Hq=32, d=128, b=16, nb=4096, dtype="torch.bfloat16")
    a = zp.compress_workspace_bytes(cache, 1, 128, 16)
    b = zp.compress_workspace_bytes(cache, 64, 128, 16)
    assert 0 < a < b and b % 256 == 0
    # tables and pointers, plus the evicted slots: L*R*H*E int32
    assert b >= 2 * 64 * 8 * 16 * 4 + 64 * 128 * 4 + 64 * 127 * 4
    # 64 requests x 8 KV heads fill the GPU: one workgroup per (request, head),
    # no split and no workspace; a single request is split in chunks of whole
    # multiples of 8 blocks, with one partial (m, l, o[d]) per split
    assert zp.paged_decode_workspace_bytes(cache, 64, 128) == 0
    assert zp.paged_decode_workspace_bytes(cache, 64, 8) == 0
    assert zp.paged_decode_workspace_bytes(cache, 1, 128) == 1 * 32 * 16 * 130 * 4


def test_decode_and_append_reject_bad_arguments():
    cache = _fake_cache()
    q = _FakeTensor((1, 4, 64), "torch.float32")
    seq = _FakeTensor((1,), "torch.int32")
    out = _FakeTensor((1, 4, 64), "torch.float32")
    tab = _FakeTensor((1, 8), "torch.int32")
    with pytest.raises(zp.ZpError):
        zp.paged_decode(cache, 1, q, tab, seq, 0.125, out, None, stream=0)      # layer out of range
    with pytest.raises(zp.ZpError):
        zp.paged_decode(cache, 0, q, tab, seq, -1.0, out, None, stream=0)       # bad scale
    tab_big = _FakeTensor((1, 64), "torch.int32")
    with pytest.raises(zp.ZpError) as e:
        zp.paged_decode(cache, 0, q, tab_big, seq, 0.125, out, None, stream=0)  # needs a workspace
    assert "workspace" in str(e.value)
    lib = zp.lib()
    assert lib.zp_append_kv(cache.ref, 3, 1, q.data_ptr(), q.data_ptr(), seq.data_ptr(), None) == \
        zp.ZP_ERR_INVALID


def test_size_limits_are_checked_before_any_work():
    """The largest shapes the kernels take are accepted; one step past any of
    them is rejected with a message (no work is ever enqueued for them)."""
    lib = zp.lib()
    c16 = _fake_cache(H=1, Hq=4, d=128, b=16, nb=1024, dtype="torch.bfloat16")
    c32 = _fake_cache(H=1, Hq=4, d=128, b=32, nb=1024, dtype="torch.bfloat16")
    c16g8 = _fake_cache(H=1, Hq=8, d=128, b=16, nb=1024, dtype="torch.bfloat16")
    ok = [(c16, 512, 512, 16),      # 8192 cached slots, one row group
          (c16g8, 256, 256, 16),    # 128 window rows at 4096 slots
          (c16, 83, 20, 16)]        # 1024 evictions per head
    bad = [(c16, 513, 513, 16, "n_max"),
           (c32, 257, 257, 32, "n_src*block_size"),
           (c16g8, 257, 257, 16, "beyond the scoring kernel"),
           (c16, 84, 20, 16, "evictions per head")]
    for c, n_src, n_max, w in ok:
        assert lib.zp_compress_workspace_bytes_n(c.ref, 1, n_src, n_max, w) > 0, zp.last_error()
    for c, n_src, n_max, w, msg in bad:
        assert lib.zp_compress_workspace_bytes_n(c.ref, 1, n_src, n_max, w) == 0
        assert msg in zp.last_error(), zp.last_error()


# ------------------------------------------------------------------ debug switches

def test_debug_flags_round_trip_and_reject_unknown_bits():
    before = zp.debug_flags()
    try:
        zp.set_debug_flags(zp.ZP_DEBUG_TRACE | zp.ZP_DEBUG_VALIDATE)
        assert zp.debug_flags() == zp.ZP_DEBUG_TRACE | zp.ZP_DEBUG_VALIDATE
        with pytest.raises(zp.ZpError):
            zp.set_debug_flags(8)
        assert zp.debug_flags() == zp.ZP_DEBUG_TRACE | zp.ZP_DEBUG_VALIDATE
        # tracing on: the planner runs inside a roctx range when a roctx
        # library is there, and without one nothing changes
        pool = zp.BlockPool(16, manual_fence=True)
        tab = pool.alloc(8).reshape(2, 4).astype(np.int32).copy()
        src, dst, freed = zp.compress_plan(pool, 4, tab)
        assert src.shape == (2, 4) and freed.size == 0
        assert isinstance(zp.trace_available(), bool)
    finally:
        zp.set_debug_flags(before)


def test_debug_flags_come_from_the_environment():
    code = ("import compressed_paged_kv_amd as zp; "
            "print(zp.debug_flags(), flush=True)")
    env = dict(os.environ, ZP_TRACE="1", ZP_DEBUG_POISON="0", ZP_VALIDATE="yes")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, check=True).stdout.strip().splitlines()[-1]
    assert int(out) == zp.ZP_DEBUG_TRACE | zp.ZP_DEBUG_VALIDATE
