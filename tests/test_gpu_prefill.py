"""GPU end-to-end run of chunked prefill through the scheduler.

Long prompts (up to 470 tokens against a budget of 128) are written one
chunk per step with zp_append_kv (one row per token).  When a chunk carries
a request past the cap, the request is compressed in the same step
(window = the chunk's last w queries), in one call with the step's other
compressions, each request with the block count it holds; a final chunk
that ends inside the window band records its window queries in a query
slot, and decode records the rest, so the compression at the cap then uses
rows from both.  Every compression (past the cap after a
chunk, and at the cap after decode) is checked against the oracle on the
cache as it stood, to the parity bar of the other GPU tests, and decode
steps against the oracle's decode.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import DECODE_ATOL, GpuRun, check_case, say
from synth.device import to_numpy, to_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_paged_kv_amd as zp
    zp.lib()


def _bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))


def test_chunked_prefill_through_compression_and_decode():
    import compressed_paged_kv_amd as zp
    dev = "cuda"
    H, Hq, d, b, n_max, w, S, chunk, nb = 2, 8, 128, 16, 8, 16, 4, 48, 160
    T, k_keep = n_max * b, (n_max - 1) * b
    geom = synth.Geometry(1, H, Hq, d, b, nb, "bf16")
    rng = np.random.default_rng(4100)
    prompts = {0: 300, 1: 90, 2: 124, 3: 470}
    say(f"[gpu prefill] prompts {prompts}, budget {T} (n_max {n_max}, b {b}), w {w}, chunk {chunk}")
    kp = to_tensor(synth.f32_to_bf16_bits(np.full((nb, H, b, d), np.nan, np.float32)), dev)
    vp = to_tensor(synth.f32_to_bf16_bits(np.full((nb, H, b, d), np.nan, np.float32)), dev)
    cache = zp.KVCache([kp], [vp], Hq)
    pool = zp.BlockPool(nb)
    sched = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=S,
                         max_running=4, prefill_chunk=chunk)
    for rid, P in prompts.items():
        sched.add(rid, P, 40)
    q_store = torch.zeros((S * w, Hq, d), dtype=torch.bfloat16, device=dev)
    lse_store = torch.zeros((S * w, Hq), dtype=torch.float32, device=dev)
    dws = torch.empty(max(max(zp.paged_decode_workspace_bytes(cache, r, n_max) for r in range(1, 5)),
                          16), dtype=torch.uint8, device=dev)
    stats = dict(chunks=0, chunk_compressions=0, cap_compressions=0, band_rows=0, decode_checks=0,
                 mixed_calls=0)
    chunks_per_req = {rid: 0 for rid in prompts}
    n_src_seen = set()
    for step in range(140):
        plan = sched.plan()
        # ---- decode (recording window rows)
        R_d = plan["decode_ids"].size
        if R_d:
            tab_d, _ = sched.tables(plan["decode_ids"])
            q = to_tensor(_bf16(rng, (R_d, Hq, d)), dev)
            kn, vn = to_tensor(_bf16(rng, (R_d, H, d)), dev), to_tensor(_bf16(rng, (R_d, H, d)), dev)
            out = torch.empty((R_d, Hq, d), dtype=torch.float32, device=dev)
            zp.append_kv(cache, 0, kn, vn, torch.from_numpy(plan["decode_slot"]).to(dev))
            zp.paged_decode(cache, 0, q, torch.from_numpy(tab_d).to(dev),
                            torch.from_numpy(plan["decode_seq_len"]).to(dev), 1.0 / np.sqrt(d), out,
                            dws, lse_out=lse_store, q_out=q_store,
                            lse_rows=torch.from_numpy(plan["decode_record_row"]).to(dev))
            if step % 5 == 0:
                torch.cuda.synchronize()
                want = oracle.decode(to_numpy(kp), to_numpy(vp), to_numpy(q), tab_d,
                                     plan["decode_seq_len"], num_q_heads=Hq)
                assert np.abs(out.cpu().numpy() - want).max() <= DECODE_ATOL
                stats["decode_checks"] += 1
        # ---- prefill chunks: K/V rows written, window-band queries recorded
        chunk_wq = {}
        for i, rid in enumerate(plan["prefill_ids"].tolist()):
            t0, n, row = (int(plan["prefill_start"][i]), int(plan["prefill_len"][i]),
                          int(plan["prefill_record_row"][i]))
            tab, _ = sched.tables([rid], width=max(n_max, (t0 + n + b - 1) // b))
            pos = np.arange(t0, t0 + n)
            slots = (tab[0, pos // b] * b + pos % b).astype(np.int32)
            kc, vc, qc = _bf16(rng, (n, H, d)), _bf16(rng, (n, H, d)), _bf16(rng, (n, Hq, d))
            zp.append_kv(cache, 0, to_tensor(kc, dev), to_tensor(vc, dev),
                         torch.from_numpy(slots).to(dev))
            if row >= 0:   # positions at or past T - w go to the query slot
                band = pos >= T - w
                q_store[row + pos[band] - (T - w)] = to_tensor(qc[band], dev)
                stats["band_rows"] += int(band.sum())
            chunk_wq[rid] = qc[n - w:] if n >= w else None   # the chunk's last w queries
            chunks_per_req[rid] += 1
            stats["chunks"] += 1
        torch.cuda.synchronize()
        # ---- compressions: one call over every request the step compresses,
        # each with its own block count (rows padded with -1)
        news = {}
        ids = plan["compress_ids"].tolist()
        if ids:
            counts = plan["compress_n_src"].astype(np.int32)
            qslots = plan["compress_qslot"].tolist()
            width = int(counts.max())
            tab, lens = sched.tables(ids, width=width)
            assert np.array_equal(lens, counts * b)
            for k in range(len(ids)):
                assert np.all(tab[k, :counts[k]] >= 0) and np.all(tab[k, counts[k]:] == -1)
            wq_h = np.empty((len(ids), w, Hq, d), dtype=np.uint16)
            for k, (rid, qs) in enumerate(zip(ids, qslots)):
                if qs >= 0:     # at the cap: the rows recorded in its query slot
                    wq_h[k] = to_numpy(q_store[qs * w:(qs + 1) * w])
                else:           # right after a chunk: its last w queries
                    assert chunk_wq[rid] is not None
                    wq_h[k] = chunk_wq[rid]
            mixed = int(counts.min()) != width
            case = synth.CompressCase(f"step{step}", 0, geom, n_max, w, tab.copy(),
                                      pool.refcounts(), [to_numpy(kp)], [to_numpy(vp)], [wq_h],
                                      [], [], [], num_blocks=counts.copy() if mixed else None)
            R_c = len(ids)
            dbg = dict(importance=torch.full((1, R_c, H, width * b), float("nan"), device=dev),
                       redundancy=torch.full((1, R_c, H, width * b), float("nan"), device=dev),
                       score=torch.full((1, R_c, H, width * b), float("nan"), device=dev),
                       kept=torch.full((1, R_c, H, k_keep), -1, dtype=torch.int32, device=dev))
            ws = torch.empty(zp.compress_workspace_bytes(cache, R_c, n_max, w, n_src=width),
                             dtype=torch.uint8, device=dev)
            freed = zp.compress(cache, pool, n_max, w, tab, [to_tensor(wq_h, dev)], ws, debug=dbg,
                                num_blocks=counts if mixed else None)
            torch.cuda.synchronize()
            run = GpuRun(tables=tab.copy(), refcounts=pool.refcounts(), freed=freed.copy(),
                         A=dbg["importance"].cpu().numpy(), R=dbg["redundancy"].cpu().numpy(),
                         s=dbg["score"].cpu().numpy(), kept=dbg["kept"].cpu().numpy(),
                         k_pool=[to_numpy(kp)], v_pool=[to_numpy(vp)], out=None,
                         appended_k=None, appended_v=None)
            check_case(case, run, check_decode=False)
            stats["mixed_calls"] += int(mixed)
            for k, rid in enumerate(ids):
                news[rid] = tab[k, :n_max].copy()
                if counts[k] > n_max:
                    stats["chunk_compressions"] += 1
                    n_src_seen.add(int(counts[k]))
                elif qslots[k] >= 0:
                    stats["cap_compressions"] += 1
                else:
                    stats["chunk_compressions"] += 1
        if plan["compress_ids"].size:
            sched.compress_commit(np.stack([news[r] for r in plan["compress_ids"].tolist()]))
        pool.sync()
        pool.fence()
        st = sched.stats()
        if st["running"] == 0 and st["waiting"] == 0:
            break
    say(f"[gpu prefill] {stats}, chunks per request {chunks_per_req}, n_src past the cap "
        f"{sorted(n_src_seen)}")
    assert chunks_per_req[3] >= 3 and stats["chunk_compressions"] >= 3
    assert len(n_src_seen) >= 2          # compressions past the cap by different amounts
    assert stats["cap_compressions"] >= 2 and stats["band_rows"] > 0
    assert stats["decode_checks"] >= 5
    assert stats["mixed_calls"] >= 1     # one call over requests holding different counts
