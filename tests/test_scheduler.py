"""Host tests of the hybrid scheduler (zp_sched_*), no GPU.

The scheduler follows the hybrid scheduling of the Zipage summaries (nl
page, Methodologie item 2; ko page, section 2.B): query slots only for
requests that will need compression, preemption of requests without a
slot first.  Compression calls are replaced by the host planner
(zp_compress_plan), which rewrites the tables exactly as zp_compress does.
"""
import numpy as np
import pytest

import compressed_paged_kv_amd as zp


def _run_compress(pool, sched, plan, n_max):
    if plan["compress_ids"].size:
        tab, lens = sched.tables(plan["compress_ids"])
        assert np.all(lens == n_max * sched.block_size)
        zp.compress_plan(pool, n_max, tab)
        sched.compress_commit(tab)


def test_config_and_request_validation():
    pool = zp.BlockPool(16, manual_fence=True)
    for bad in (dict(n_max=1), dict(block_size=8), dict(window=0), dict(window=17),
                dict(num_query_slots=0), dict(max_running=0)):
        kw = dict(n_max=4, block_size=16, window=4, num_query_slots=1, max_running=4)
        kw.update(bad)
        with pytest.raises(zp.ZpError):
            zp.Scheduler(pool, **kw)
    s = zp.Scheduler(pool, n_max=4, block_size=16, window=4, num_query_slots=1, max_running=4)
    s.add(1, 60, 5)                       # 60 = 4*16 - 4, the longest prompt
    with pytest.raises(zp.ZpError):
        s.add(1, 10, 5)                   # duplicate id
    with pytest.raises(zp.ZpError):
        s.add(2, 61, 5)                   # prompt reaching into the window
    with pytest.raises(zp.ZpError):
        s.add(3, 10, 0)


def test_window_rows_slot_and_compression_cycle():
    """One request: no slot until its next token is in the window, rows
    0..w-1 recorded in order, compression at the cap, back to K_keep."""
    n_max, b, w = 3, 16, 4
    T = n_max * b
    pool = zp.BlockPool(8, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=2, max_running=4)
    s.add(7, 40, 1000)
    p = s.plan()
    assert p["admitted"].tolist() == [7]
    tab, lens = s.tables([7])
    assert lens.tolist() == [40] and (tab[0, :3] >= 0).all()
    rows, seen_compress = [], 0
    for step in range(30):
        p = s.plan()
        pool.fence()
        if p["compress_ids"].size:
            assert p["decode_ids"].size == 0
            assert rows == [p["compress_qslot"][0] * w + i for i in range(w)]
            rows = []
            seen_compress += 1
            _run_compress(pool, s, p, n_max)
            assert s.tables([7])[1].tolist() == [(n_max - 1) * b]
            assert s.stats()["free_query_slots"] == 2
            continue
        assert p["decode_ids"].tolist() == [7]
        seq = int(p["decode_seq_len"][0])
        pos = seq - 1
        row = int(p["decode_record_row"][0])
        if pos >= T - w:
            assert row >= 0 and row % w == pos - (T - w)
            rows.append(row)
        else:
            assert row == -1
        # the new token's slot is in the block holding position pos
        tab, _ = s.tables([7])
        assert p["decode_slot"][0] == tab[0, pos // b] * b + pos % b
    assert seen_compress >= 2


def test_query_slots_are_limited_and_waiting_requests_stall():
    n_max, b, w = 2, 16, 4
    pool = zp.BlockPool(20, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=1, max_running=4)
    s.add(0, 28, 100)
    s.add(1, 28, 100)
    s.plan()
    p = s.plan()                            # both decode position 28 (window starts at 28)
    assert p["decode_ids"].tolist() == [0]  # only one slot: request 1 waits
    assert p["decode_record_row"].tolist() == [0]
    for _ in range(3):
        p = s.plan()
        assert p["decode_ids"].tolist() == [0]
    p = s.plan()                            # request 0 at the cap compresses
    assert p["compress_ids"].tolist() == [0] and p["decode_ids"].tolist() == []
    _run_compress(pool, s, p, n_max)
    p = s.plan()                            # the slot is free again: request 1 takes it
    assert 1 in p["decode_ids"].tolist()


def test_preemption_takes_the_last_admitted_slotless_request_possibly_itself():
    n_max, b, w = 4, 16, 4
    # 0 (1 block), 1 (1 block), 2 (4 blocks, next token 60 in the window):
    # the pool is full; 0 needs a block at position 16
    pool = zp.BlockPool(6, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=1, max_running=4)
    s.add(0, 16, 100)
    s.add(1, 10, 100)
    s.add(2, 60, 100)
    p = s.plan()
    assert p["admitted"].tolist() == [0, 1, 2] and pool.num_free() == 0
    p = s.plan()
    # 0 waits and preempts 1 (no slot, admitted after 0); 1 drops out; 2 takes
    # the slot and decodes in its window
    assert p["preempted"].tolist() == [1]
    assert p["decode_ids"].tolist() == [2] and p["decode_record_row"].tolist() == [0]
    pool.fence()
    p = s.plan()                      # the block 1 gave back goes to 0
    assert 0 in p["decode_ids"].tolist() and p["preempted"].size == 0


def test_preemption_spares_slot_holders_when_a_slotless_request_exists():
    n_max, b, w = 4, 16, 4
    # 2 (slot holder, admitted last) and 0 (no slot, admitted first): when 1
    # needs a block the victim is 1 itself (no slot, admitted after 0), not 2
    pool = zp.BlockPool(6, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=1, max_running=4)
    s.add(0, 10, 100)
    s.add(1, 16, 100)
    s.add(2, 60, 100)
    s.plan()
    p = s.plan()
    assert p["preempted"].tolist() == [1]
    assert sorted(p["decode_ids"].tolist()) == [0, 2]
    # with only slot holders left, the last admitted one goes
    pool2 = zp.BlockPool(8, manual_fence=True)
    s2 = zp.Scheduler(pool2, n_max=n_max, block_size=b, window=w, num_query_slots=2,
                      max_running=4)
    s2.add(0, 60, 100)
    s2.add(1, 60, 100)
    s2.plan()
    p = s2.plan()                      # both take slots, decode 60
    assert sorted(p["decode_ids"].tolist()) == [0, 1]
    for _ in range(3):
        p = s2.plan()
    # both at the cap now: compress, then position 48 starts no block... they
    # reach 64 = N_max*b only via compression; no preemption ever needed
    assert p["compress_ids"].size == 0 or p["preempted"].size == 0


@pytest.mark.parametrize("seed", range(12))
def test_random_workload_invariants_and_completion(seed):
    rng = np.random.default_rng(seed)
    n_max, b, w = int(rng.integers(3, 7)), 16, int(rng.choice([4, 16]))
    T = n_max * b
    nblocks = int(rng.integers(3 * n_max, 6 * n_max))
    S = int(rng.integers(1, 4))
    pool = zp.BlockPool(nblocks, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=S,
                     max_running=int(rng.integers(2, 9)))
    R = 30
    for i in range(R):
        s.add(i, int(rng.integers(1, T - w + 1)), int(rng.integers(1, 3 * T)))
    done, recorded = set(), {}
    for step in range(20000):
        p = s.plan()
        done |= set(p["finished"].tolist())
        for r in p["preempted"].tolist() + p["finished"].tolist():
            recorded.pop(r, None)  # their slot is free again
        live = [int(x) for x in np.concatenate([p["decode_ids"], p["compress_ids"]])]
        if live:
            tab, lens = s.tables(live, width=n_max + 2)
            assert np.all(tab[:, n_max:] == -1)   # never more than n_max blocks
            for i, r in enumerate(live):
                nb = int((tab[i] >= 0).sum())
                assert nb <= n_max
                assert nb in ((lens[i] + b - 1) // b, n_max)
        # decodes listed longest first, each entry's slot the token's place in its table
        assert np.all(np.diff(p["decode_seq_len"]) <= 0)
        if p["decode_ids"].size:
            tab_d, _ = s.tables(p["decode_ids"], width=n_max)
            pos = p["decode_seq_len"] - 1
            want = tab_d[np.arange(len(pos)), pos // b] * b + pos % b
            np.testing.assert_array_equal(p["decode_slot"], want)
        # query-slot rows: recorded in window order, exactly w before compression
        for r, row, seq in zip(p["decode_ids"].tolist(), p["decode_record_row"].tolist(),
                               p["decode_seq_len"].tolist()):
            pos = seq - 1
            if pos >= T - w:
                assert row >= 0 and row % w == pos - (T - w) and row // w < S
                recorded.setdefault(r, []).append(row)
            else:
                assert row == -1
        for r, slot in zip(p["compress_ids"].tolist(), p["compress_qslot"].tolist()):
            assert recorded.pop(r) == [slot * w + i for i in range(w)]
        # no two requests record into the same slot at once
        slots = [v[0] // w for v in recorded.values() if v]
        assert len(slots) == len(set(slots))
        _run_compress(pool, s, p, n_max)
        pool.fence()
        # every block in use belongs to exactly one table
        rc = pool.refcounts()
        assert rc.max() <= 1
        if len(done) == R:
            break
    assert len(done) == R, f"only {len(done)} of {R} finished"
    assert pool.num_free() == nblocks


# ------------------------------------------------------------------ chunked prefill

def _drive_prefill(s, pool, n_max, steps, on_step=None):
    """Run plans; compress (host planner, per n_src group) and commit each
    step's compressions; return the per-step plans."""
    plans = []
    for _ in range(steps):
        p = s.plan()
        if on_step:
            on_step(p)
        if p["compress_ids"].size:
            news = []
            for i, rid in enumerate(p["compress_ids"]):
                n_src = int(p["compress_n_src"][i])
                tab, lens = s.tables([rid], width=n_src)
                assert lens.tolist() == [n_src * s.block_size]
                assert np.all(tab[0] >= 0)                 # every block held, all full
                zp.compress_plan(pool, n_max, tab)
                news.append(tab[0, :n_max])
            s.compress_commit(np.stack(news))
        pool.fence()
        plans.append(p)
    return plans


def test_chunked_prefill_validation():
    pool = zp.BlockPool(64, manual_fence=True)
    kw = dict(n_max=8, block_size=16, window=16, num_query_slots=2, max_running=4)
    for bad in (-16, 24, 16 * 600):           # negative, not a multiple of b, past the limits
        with pytest.raises(zp.ZpError):
            zp.Scheduler(pool, prefill_chunk=bad, **kw)
    s = zp.Scheduler(pool, prefill_chunk=48, **kw)
    s.add(1, 5000, 3)                          # any prompt length with chunked prefill
    with pytest.raises(zp.ZpError):
        s.add(2, 0, 3)


def test_chunked_prefill_of_a_long_prompt():
    """n_max = 8, b = 16 (T = 128), w = 16, chunks of 48, a 300-token prompt.
    Worked by hand from the rule in the header: chunks 0..47, 48..95 (the
    cache ends at 96 <= T - w = 112); then 96 + 48 = 144 > 112 and the rest
    reaches T, so the chunk ends at the block boundary 144: compress 9 blocks
    -> 112; then 112 + 48 = 160, boundary 160: 10 blocks -> 112, twice
    (prompt tokens 144..191 and 192..239); then 48 tokens are left: 112 + 48
    = 160 again (10 blocks) -> 112 with 12 left; 112 + 12 = 124 lies in the
    window band (112, 128): written whole, positions 112..123 recorded in
    query-slot rows 0..11, and decode goes on from 124: positions 124..127
    recorded in rows 12..15, then the cap compression (8 blocks)."""
    n_max, b, w = 8, 16, 16
    pool = zp.BlockPool(64, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=1, max_running=2,
                     prefill_chunk=48)
    s.add(5, 300, 10)
    chunks, comps, rows = [], [], []

    def look(p):
        for i in range(p["prefill_ids"].size):
            chunks.append((int(p["prefill_start"][i]), int(p["prefill_len"][i]),
                           int(p["prefill_record_row"][i])))
        for i in range(p["compress_ids"].size):
            comps.append(int(p["compress_n_src"][i]))
            assert p["compress_qslot"][i] == (-1 if p["prefill_ids"].size else 0)
        for i in range(p["decode_ids"].size):
            rows.append(int(p["decode_record_row"][i]))
        # a request writes a chunk or decodes, never both in one step
        assert not (set(p["prefill_ids"].tolist()) & set(p["decode_ids"].tolist()))

    _drive_prefill(s, pool, n_max, 12, look)
    assert chunks == [(0, 48, -1), (48, 48, -1), (96, 48, -1), (112, 48, -1), (112, 48, -1),
                      (112, 48, -1), (112, 12, 0)]
    assert comps == [9, 10, 10, 10, 8]
    # decode after the prefill: 124..127 in rows 12..15, then the cap, then
    # 112.. again outside the window
    assert rows[:4] == [12, 13, 14, 15] and rows[4:] == [-1] * (len(rows) - 4)
    tab, lens = s.tables([5])
    assert int(lens[0]) == 112 + len(rows) - 4
    # every block held is counted once, the rest of the pool free
    assert sum(pool.refcount(i) for i in range(64)) == int((tab[0] >= 0).sum())


def test_chunked_prefill_batch_by_hand():
    """n_max = 8, b = 16 (T = 128, K_keep = 112), w = 8 (window start 120),
    chunks of 64; four requests admitted together, worked by hand:
      1: 200 tokens: (0, 64); (64, 64) ends at 128 = T -> compress 8 blocks;
         (112, 64) ends at 176, a block boundary -> compress 11; (112, 8)
         ends at 120 <= 120, plain; then decodes from 120 with a query slot.
      2: 30 tokens: (0, 30), then decodes.
      3: 124 tokens: (0, 64); (64, 60) ends at 124, inside the band
         (120, 128) with no more prompt to reach T: written whole with its
         positions 120..123 in query-slot rows 0..3 (slot 0), then decodes
         124.. into rows 4..7.
      4: 150 tokens: (0, 64); (64, 64) -> compress 8; then 22 left: 112 + 22
         = 134 floors to the boundary 128 -> (112, 16), compress 8; (112, 6)
         plain; decodes from 118."""
    n_max, b, w = 8, 16, 8
    pool = zp.BlockPool(64, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=4, max_running=4,
                     prefill_chunk=64)
    for rid, P in ((1, 200), (2, 30), (3, 124), (4, 150)):
        s.add(rid, P, 50)
    seen = []

    def look(p):
        pre = {int(i): (int(a), int(l), int(r)) for i, a, l, r in
               zip(p["prefill_ids"], p["prefill_start"], p["prefill_len"], p["prefill_record_row"])}
        comp = dict(zip(p["compress_ids"].tolist(), p["compress_n_src"].tolist()))
        dec = {int(i): (int(l) - 1, int(r)) for i, l, r in
               zip(p["decode_ids"], p["decode_seq_len"], p["decode_record_row"])}
        seen.append((pre, comp, dec))

    _drive_prefill(s, pool, n_max, 5, look)
    assert seen[0] == ({1: (0, 64, -1), 2: (0, 30, -1), 3: (0, 64, -1), 4: (0, 64, -1)}, {}, {})
    assert seen[1] == ({1: (64, 64, -1), 3: (64, 60, 0), 4: (64, 64, -1)}, {1: 8, 4: 8},
                       {2: (30, -1)})
    assert seen[2] == ({1: (112, 64, -1), 4: (112, 16, -1)}, {1: 11, 4: 8},
                       {2: (31, -1), 3: (124, 4)})
    assert seen[3] == ({1: (112, 8, -1), 4: (112, 6, -1)}, {}, {2: (32, -1), 3: (125, 5)})
    assert seen[4] == ({}, {}, {1: (120, 8), 2: (33, -1), 3: (126, 6), 4: (118, -1)})
    tab, lens = s.tables([1, 2, 3, 4], width=n_max)
    assert lens.tolist() == [121, 34, 127, 119]
    assert sum(pool.refcount(i) for i in range(64)) == int((tab >= 0).sum())


def test_chunked_prefill_waits_for_blocks_and_preempts():
    """A pool too small for two long prompts: the second request's chunk
    finds no block, preempts the last-admitted request without a query slot
    (itself here), and restarts its prefill from the queue later."""
    n_max, b, w = 4, 16, 16
    pool = zp.BlockPool(9, manual_fence=True)
    s = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=2, max_running=2,
                     prefill_chunk=32)
    s.add(1, 100, 3)
    s.add(2, 100, 3)
    preempted = []
    plans = _drive_prefill(s, pool, n_max, 12, lambda p: preempted.extend(p["preempted"].tolist()))
    assert 2 in preempted
    # everything either finished or still holds consistent counts
    held = sum(pool.refcount(i) for i in range(9))
    ids = [r for r in (1, 2)]
    tab, _ = s.tables(ids, width=n_max + 2)
    assert held == int((tab >= 0).sum())
