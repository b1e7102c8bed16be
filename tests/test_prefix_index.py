"""Host tests of the prefix index (zp_prefix_*), no GPU.

Full prompt blocks are listed by their tokens and the blocks before them;
a new request matching a listed prefix shares those physical blocks
(reference counts, the paged-cache guide's "How it works"), and a listed
block counts as shared, so compression re-targets instead of rewriting it
(ko page section 2.C).
"""
import numpy as np
import pytest

import compressed_paged_kv_amd as zp


def _pool_with(n, allocated):
    pool = zp.BlockPool(n, manual_fence=True)
    ids = np.zeros(allocated, dtype=np.int32)
    zp.lib().zp_block_alloc(pool.handle, allocated, ids.ctypes.data_as(zp._binding._i32p))
    return pool, ids


def test_insert_match_longest_full_block_prefix():
    b = 4
    pool, ids = _pool_with(20, 3)
    ix = zp.PrefixIndex(pool, b)
    toks = np.arange(100, 111)                     # 11 tokens: 2 full blocks + 3
    assert ix.insert(toks, ids) == 2 and len(ix) == 2
    assert pool.refcount(int(ids[0])) == 2 and pool.refcount(int(ids[2])) == 1
    # same first 9 tokens: both full blocks match; each matched block gains a reference
    m = ix.match(np.concatenate([toks[:9], [7, 7, 7]]))
    assert m.tolist() == ids[:2].tolist()
    assert pool.refcount(int(ids[0])) == 3
    # a change inside block 1 stops the match after block 0
    other = toks.copy()
    other[5] = -1
    assert ix.match(other).tolist() == ids[:1].tolist()
    # a change in block 0 matches nothing, even if block 1's tokens are equal
    other = toks.copy()
    other[0] = -1
    assert ix.match(other).size == 0
    # fewer tokens than a block: nothing
    assert ix.match(toks[:3]).size == 0


def test_same_block_tokens_after_different_prefixes_are_different_entries():
    b = 2
    pool, ids = _pool_with(10, 4)
    ix = zp.PrefixIndex(pool, b)
    ix.insert([1, 2, 9, 9], ids[:2])
    ix.insert([3, 4, 9, 9], ids[2:4])
    assert ix.match([1, 2, 9, 9]).tolist() == ids[:2].tolist()
    assert ix.match([3, 4, 9, 9]).tolist() == ids[2:4].tolist()
    # inserting an already listed prefix keeps the first blocks
    pool2_ids = ids[2:4]
    assert ix.insert([1, 2, 9, 9], pool2_ids) == 0
    assert ix.match([1, 2, 9, 9]).tolist() == ids[:2].tolist()


def test_evict_drops_least_recently_used_leaves_and_frees_unheld_blocks():
    b = 2
    pool, ids = _pool_with(12, 3)
    ix = zp.PrefixIndex(pool, b)
    ix.insert([1, 1, 2, 2, 3, 3], ids)
    # the request that filled them is done: give back its references
    freed = np.zeros(3, dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    zp.lib().zp_block_release(pool.handle, ids.ctypes.data_as(zp._binding._i32p), 3,
                              freed.ctypes.data_as(zp._binding._i32p),
                              n.ctypes.data_as(zp._binding._i32p))
    assert n[0] == 0                       # still held by the index
    before = pool.num_free()
    out = ix.evict(1)                      # only the leaf (block 2) can go first
    assert out.tolist() == [int(ids[2])] and pool.num_free() == before + 1
    assert ix.match([1, 1, 2, 2, 3, 3]).tolist() == ids[:2].tolist()
    # the matched blocks are held by the caller now: evicting them frees nothing
    out = ix.evict(5)
    assert out.size == 0 and len(ix) == 0
    assert pool.refcount(int(ids[0])) == 1 and pool.refcount(int(ids[1])) == 1


def test_listed_blocks_are_retargeted_by_compression_planning():
    """A request whose prompt blocks are listed compresses into new target
    blocks: the listed blocks keep their contents for later matches."""
    b, n_max = 4, 3
    pool, ids = _pool_with(20, n_max)
    ix = zp.PrefixIndex(pool, b)
    toks = np.arange(n_max * b)
    ix.insert(toks, ids)
    tab = ids[None, :].copy()
    src, dst, freed = zp.compress_plan(pool, n_max, tab)
    assert not np.any(np.isin(tab[0], ids))        # every position re-targeted
    assert freed.size == 0                          # the index still holds them
    assert ix.match(toks).tolist() == ids.tolist()


def test_invalid_insert_changes_nothing():
    pool, ids = _pool_with(8, 1)
    ix = zp.PrefixIndex(pool, 2)
    with pytest.raises(zp.ZpError):
        ix.insert([1, 2, 3, 4], [int(ids[0]), 7])    # block 7 is not allocated
    assert len(ix) == 0 and pool.refcount(int(ids[0])) == 1
