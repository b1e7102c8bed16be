"""GPU end-to-end run of the hybrid scheduler with recorded query slots.

A small continuous-batching run: the scheduler plans every step; decode
appends each request's token and records, while the request is in its
observation window, its query and log-sum-exp into its query-slot rows;
requests at the cap are compressed from exactly those recorded rows and
normalisers, on alternate calls read in place from the query-slot stores
(window_slots) or gathered per request first.  Every compression is
checked against the oracle run on the cache as it stood (the window queries
read back from the slots) to the parity bar of the other GPU tests, and
sampled decode steps against the oracle's decode.
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


@pytest.mark.parametrize("w,nb", [(8, 48), (16, 48), (8, 22)])
def test_scheduler_driven_run_matches_oracle(w, nb):
    """nb = 22 blocks cannot hold six requests at the cap (30 blocks): the
    run goes through preemptions (recompute), and the requests that keep
    running still match the oracle."""
    import compressed_paged_kv_amd as zp
    dev = "cuda"
    H, Hq, d, b, n_max, S = 2, 4, 64, 16, 5, 4
    T = n_max * b
    geom = synth.Geometry(1, H, Hq, d, b, nb, "bf16")
    rng = np.random.default_rng(300 + w)
    say(f"[gpu continuous] scheduler-driven run, w={w}, n_max={n_max}, pool {nb}")
    n_preempted = 0
    kp_h = synth.f32_to_bf16_bits(rng.standard_normal((nb, H, b, d)).astype(np.float32))
    vp_h = synth.f32_to_bf16_bits(rng.standard_normal((nb, H, b, d)).astype(np.float32))
    kp, vp = to_tensor(kp_h, dev), to_tensor(vp_h, dev)
    cache = zp.KVCache([kp], [vp], Hq)
    pool = zp.BlockPool(nb)
    sched = zp.Scheduler(pool, n_max=n_max, block_size=b, window=w, num_query_slots=S,
                         max_running=6)
    for i in range(6):
        sched.add(i, int(rng.integers(40, T - w + 1)), int(rng.integers(30, 90)))
    q_store = torch.zeros((S * w, Hq, d), dtype=torch.bfloat16, device=dev)
    lse_store = torch.zeros((S * w, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(zp.compress_workspace_bytes(cache, S, n_max, w), dtype=torch.uint8,
                     device=dev)
    dws = torch.empty(max(max(zp.paged_decode_workspace_bytes(cache, r, n_max)
                              for r in range(1, 7)), 16), dtype=torch.uint8, device=dev)
    n_compressions = n_decode_checks = n_in_place = n_calls = 0
    for step in range(160):
        plan = sched.plan()
        n_preempted += plan["preempted"].size
        R_d, R_c = plan["decode_ids"].size, plan["compress_ids"].size
        if R_c:
            ids = plan["compress_ids"]
            tab, lens = sched.tables(ids)
            rows = torch.from_numpy(plan["compress_qslot"].astype(np.int64)).to(dev)
            wq = q_store.view(S, w, Hq, d).index_select(0, rows).contiguous()
            wl = lse_store.view(S, w, Hq).index_select(0, rows).contiguous()
            case = synth.CompressCase(f"step{step}", 0, geom, n_max, w, tab.copy(),
                                      pool.refcounts(), [to_numpy(kp)], [to_numpy(vp)],
                                      [to_numpy(wq)], [], [], [])
            k_keep = (n_max - 1) * b
            dbg = dict(importance=torch.full((1, R_c, H, T), float("nan"), device=dev),
                       redundancy=torch.full((1, R_c, H, T), float("nan"), device=dev),
                       score=torch.full((1, R_c, H, T), float("nan"), device=dev),
                       kept=torch.full((1, R_c, H, k_keep), -1, dtype=torch.int32, device=dev))
            if n_calls % 2:   # the window rows gathered per request
                freed = zp.compress(cache, pool, n_max, w, tab, [wq], ws, debug=dbg, window_lse=[wl])
            else:          # read in place from the query-slot stores
                slots = torch.from_numpy(plan["compress_qslot"].astype(np.int32)).to(dev)
                freed = zp.compress(cache, pool, n_max, w, tab, [q_store], ws, debug=dbg,
                                    window_lse=[lse_store], window_slots=slots)
                n_in_place += 1
            n_calls += 1
            torch.cuda.synchronize()
            run = GpuRun(tables=tab.copy(), refcounts=pool.refcounts(), freed=freed.copy(),
                         A=dbg["importance"].cpu().numpy(), R=dbg["redundancy"].cpu().numpy(),
                         s=dbg["score"].cpu().numpy(), kept=dbg["kept"].cpu().numpy(),
                         k_pool=[to_numpy(kp)], v_pool=[to_numpy(vp)], out=None,
                         appended_k=None, appended_v=None)
            check_case(case, run, check_decode=False)
            sched.compress_commit(tab)
            n_compressions += R_c
        if R_d:
            tab_d, _ = sched.tables(plan["decode_ids"])
            q = to_tensor(synth.f32_to_bf16_bits(
                rng.standard_normal((R_d, Hq, d)).astype(np.float32)), dev)
            kn = to_tensor(synth.f32_to_bf16_bits(
                rng.standard_normal((R_d, H, d)).astype(np.float32)), dev)
            vn = to_tensor(synth.f32_to_bf16_bits(
                rng.standard_normal((R_d, H, d)).astype(np.float32)), dev)
            slot_t = torch.from_numpy(plan["decode_slot"]).to(dev)
            seq_t = torch.from_numpy(plan["decode_seq_len"]).to(dev)
            row_t = torch.from_numpy(plan["decode_record_row"]).to(dev)
            tab_t = torch.from_numpy(tab_d).to(dev)
            out = torch.empty((R_d, Hq, d), dtype=torch.float32, device=dev)
            zp.append_kv(cache, 0, kn, vn, slot_t)
            zp.paged_decode(cache, 0, q, tab_t, seq_t, 1.0 / np.sqrt(d), out, dws,
                            lse_out=lse_store, q_out=q_store, lse_rows=row_t)
            torch.cuda.synchronize()
            if step % 7 == 0:
                want = oracle.decode(to_numpy(kp), to_numpy(vp), to_numpy(q), tab_d,
                                     plan["decode_seq_len"], num_q_heads=Hq)
                assert np.abs(out.cpu().numpy() - want).max() <= DECODE_ATOL
                n_decode_checks += 1
        pool.fence()
    say(f"[gpu continuous] w={w}, pool {nb}: {n_compressions} compressions and "
        f"{n_decode_checks} decode steps matched the oracle, {n_preempted} preemptions")
    assert n_compressions >= 3 and n_decode_checks >= 10 and n_in_place >= 1
    assert (n_preempted > 0) == (nb < 30)
