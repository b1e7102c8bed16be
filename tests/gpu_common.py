"""Helpers for the GPU parity tests: run a synthetic case through the HIP
library and compare every output with the CPU oracle.

Tolerances (fixed by the task's parity contract):
  * importance A and combined score s: |gpu - cpu| <= 1e-3 |cpu| + 1e-30;
  * redundancy R: |gpu - cpu| <= 1e-3 absolute (it crosses zero);
  * survivor sets: the GPU decision must be exactly what the oracle's
    selection rule gives on the GPU's own float32 scores, and may differ
    from the oracle's fp64 decision only at slots whose oracle score is
    within 1e-4 (relative) of the oracle's K_sel-th largest score;
  * compacted K/V: bit-exact copies of the source rows the GPU kept;
  * tables, refcounts, freed ids: exact;
  * decode output: |gpu - cpu| <= 2e-3 absolute (float32 output, bf16 or
    float32 inputs, float32 accumulation on the GPU, double in the oracle).
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np
import torch

import compressed_paged_kv_amd as zp
import oracle
from synth.device import to_numpy, to_tensor

A_RTOL, S_RTOL, FLOOR = 1e-3, 1e-3, 1e-30
R_ATOL = 1e-3
TIE_RTOL = 1e-4
DECODE_ATOL = 2e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class GpuRun:
    tables: np.ndarray
    refcounts: np.ndarray
    freed: np.ndarray
    A: np.ndarray        # [L][R][H][T]
    R: np.ndarray
    s: np.ndarray
    kept: np.ndarray     # [L][R][H][K_keep]
    k_pool: list         # host copies after compression
    v_pool: list
    out: np.ndarray      # decode output [L][R][Hq][d]
    appended_k: list     # host pools after the append (for the decode check)
    appended_v: list
    times: np.ndarray = None  # [L][R][H][5] phase wall-clock stamps, when asked for


def window_lse_on_gpu(cache, case, kp_tensors, wq_tensors, device="cuda"):
    """Normalisers of the window rows as the decode steps that produced the
    window queries record them: for window position i, zp_paged_decode_lse
    of query i over slots 0..T_r-w+i, written to row r*w + i of a [R*w][Hq]
    buffer per layer (returned as [R][w][Hq] views)."""
    g = case.geom
    R, w, n_src, b = case.num_reqs, case.window, case.n_src, g.block_size
    counts = getattr(case, "num_blocks", None)
    # each request's own length T_r (requests may hold different block counts)
    T = torch.from_numpy((np.full(R, n_src) if counts is None else counts).astype(np.int32) * b)
    T = T.to(device)
    tab_t = torch.from_numpy(np.ascontiguousarray(case.tables)).to(device)
    dws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, n_src), 16),
                      dtype=torch.uint8, device=device)
    out = torch.empty((R, g.num_q_heads, g.head_dim), dtype=torch.float32, device=device)
    res = []
    for layer in range(g.num_layers):
        buf = torch.full((R * w, g.num_q_heads), float("nan"), dtype=torch.float32, device=device)
        for i in range(w):
            seq = (T - w + i + 1).to(torch.int32).contiguous()
            rows = (torch.arange(R, dtype=torch.int32, device=device) * w + i).contiguous()
            q_i = wq_tensors[layer][:, i].contiguous()
            zp.paged_decode(cache, layer, q_i, tab_t, seq, 1.0 / np.sqrt(g.head_dim), out, dws,
                            lse_out=buf, lse_rows=rows)
        res.append(buf.view(R, w, g.num_q_heads))
    torch.cuda.synchronize()
    return res


def run_case(case, device="cuda", decode=True, recorded_lse=False, keep_prefix=False,
             device_tables=False, slot_store=None, phase_times=False) -> GpuRun:
    """``recorded_lse``: compress with the window rows' normalisers taken
    from zp_paged_decode_lse (the single-read scoring) instead of the
    self-contained two-pass scoring.  ``device_tables``: zp_compress_ex with
    a device copy of the tables (no upload when the plan is in place).
    ``slot_store`` (a seed): the window rows (and normalisers) sit in
    query-slot stores of R + 3 slots, request r's at a seeded permuted slot,
    every other slot NaN, and the call reads them in place (window_slots)."""
    g = case.geom
    L, H, b, n_max, w = g.num_layers, g.num_kv_heads, g.block_size, case.n_max, case.window
    R, n_src = case.num_reqs, case.n_src
    T, k_keep = n_src * b, (n_max - 1) * b
    kp = [to_tensor(x, device) for x in case.k_pool]
    vp = [to_tensor(x, device) for x in case.v_pool]
    wq = [to_tensor(x, device) for x in case.window_q]
    cache = zp.KVCache(kp, vp, g.num_q_heads)
    pool = zp.BlockPool.from_refcounts(case.refcounts)
    tables = case.tables.copy()
    ws = torch.empty(zp.compress_workspace_bytes(cache, R, n_max, w, n_src=n_src),
                     dtype=torch.uint8, device=device)
    dbg = dict(importance=torch.full((L, R, H, T), float("nan"), device=device),
               redundancy=torch.full((L, R, H, T), float("nan"), device=device),
               score=torch.full((L, R, H, T), float("nan"), device=device),
               kept=torch.full((L, R, H, k_keep), -1, dtype=torch.int32, device=device))
    if phase_times:
        dbg["phase_times"] = torch.zeros((L, R, H, 5), dtype=torch.int64, device=device)
    wl = window_lse_on_gpu(cache, case, kp, wq, device) if recorded_lse else None
    dtab = torch.from_numpy(np.ascontiguousarray(case.tables)).to(device) if device_tables else None
    slots_t = None
    if slot_store is not None:
        S = R + 3
        slots = np.random.default_rng(slot_store).permutation(S)[:R].astype(np.int32)
        slots_t = torch.from_numpy(slots).to(device)
        idx = torch.from_numpy(slots.astype(np.int64)).to(device)
        stores = []
        for q in wq:
            st = torch.full((S, w, g.num_q_heads, g.head_dim), float("nan"), device=device).to(q.dtype)
            st.index_copy_(0, idx, q)
            stores.append(st.view(S * w, g.num_q_heads, g.head_dim))
        wq = stores
        if wl is not None:
            lstores = []
            for x in wl:
                st = torch.full((S, w, g.num_q_heads), float("nan"), dtype=torch.float32, device=device)
                st.index_copy_(0, idx, x.contiguous())
                lstores.append(st.view(S * w, g.num_q_heads))
            wl = lstores
    freed = zp.compress(cache, pool, n_max, w, tables, wq, ws, debug=dbg, window_lse=wl,
                        keep_prefix=keep_prefix, device_tables=dtab,
                        num_blocks=getattr(case, "num_blocks", None), window_slots=slots_t)
    torch.cuda.synchronize()
    run = GpuRun(tables=tables.copy(), refcounts=pool.refcounts(), freed=freed.copy(),
                 A=dbg["importance"].cpu().numpy(), R=dbg["redundancy"].cpu().numpy(),
                 s=dbg["score"].cpu().numpy(), kept=dbg["kept"].cpu().numpy(),
                 k_pool=[to_numpy(t) for t in kp], v_pool=[to_numpy(t) for t in vp],
                 out=None, appended_k=None, appended_v=None,
                 times=dbg["phase_times"].cpu().numpy() if phase_times else None)
    if decode:
        # poison the reserved blocks' slots past the one about to be appended:
        # a decode that strayed past the length would turn its output NaN
        reserved = torch.from_numpy(tables[:, n_max - 1].astype(np.int64)).to(device)
        for layer in range(L):
            for t in (kp[layer], vp[layer]):
                t[reserved, :, 1:, :] = float("nan")
        slot = tables[:, k_keep // b] * b + k_keep % b
        slot_t = torch.from_numpy(slot.astype(np.int32)).to(device)
        tab_t = torch.from_numpy(np.ascontiguousarray(tables[:, :n_max])).to(device)
        seq = torch.full((R,), k_keep + 1, dtype=torch.int32, device=device)
        dws_bytes = zp.paged_decode_workspace_bytes(cache, R, n_max)
        dws = torch.empty(max(dws_bytes, 16), dtype=torch.uint8, device=device)
        outs = []
        for layer in range(L):
            zp.append_kv(cache, layer, to_tensor(case.k_new[layer], device),
                         to_tensor(case.v_new[layer], device), slot_t)
            out = torch.empty((R, g.num_q_heads, g.head_dim), dtype=torch.float32, device=device)
            zp.paged_decode(cache, layer, to_tensor(case.q_new[layer], device), tab_t, seq,
                            1.0 / np.sqrt(g.head_dim), out, dws)
            outs.append(out)
        torch.cuda.synchronize()
        run.out = np.stack([o.cpu().numpy() for o in outs])
        run.appended_k = [to_numpy(t) for t in kp]
        run.appended_v = [to_numpy(t) for t in vp]
    pool.sync()
    return run


def words(pool: np.ndarray) -> np.ndarray:
    """A [nb][H][b][d] pool viewed as 64-bit words per row (bit patterns)."""
    nb, H, b, d = pool.shape
    return np.ascontiguousarray(pool).view(np.uint64).reshape(nb, H, b, -1)


def rel_ok(got, want, rtol, floor=FLOOR):
    return np.abs(got - want) <= rtol * np.abs(want) + floor


def check_case(case, run: GpuRun, *, check_decode=True, layers=None, keep_prefix=False) -> dict:
    """Compare one GPU run with the oracle; raises AssertionError on failure.
    Returns a few statistics for the log."""
    g = case.geom
    b, n_max, w = g.block_size, case.n_max, case.window
    T, k_keep = case.n_src * b, (n_max - 1) * b
    C, k_sel = T - w, k_keep - w
    layers = list(range(g.num_layers)) if layers is None else layers
    ref = oracle.compress(case, layers=layers, with_pools=False, keep_prefix=keep_prefix)
    # bookkeeping, exact
    np.testing.assert_array_equal(run.tables, ref.plan.tables)
    np.testing.assert_array_equal(run.refcounts, ref.plan.refcounts)
    np.testing.assert_array_equal(np.sort(run.freed), np.sort(ref.plan.freed))
    stats = dict(max_rel_A=0.0, max_abs_R=0.0, max_rel_s=0.0, near_tie_diffs=0, max_abs_out=0.0)
    dst_blocks = set(ref.plan.dst.reshape(-1).tolist())
    nbk = getattr(case, "num_blocks", None)
    for li, layer in enumerate(layers):
        A, Rr, s = run.A[layer], run.R[layer], run.s[layer]
        Ao, Ro, so = ref.A[li], ref.R[li], ref.s[li]
        if nbk is not None:
            _check_ragged_unit_scores(A, Rr, s, Ao, Ro, so, run.kept[layer], ref.kept[li],
                                      nbk * b, w, k_sel, layer, stats)
        else:
            _check_unit_scores_uniform(A, Rr, s, Ao, Ro, so, run.kept[layer], ref.kept[li], C, w,
                                       k_sel, layer, stats)
        kept = run.kept[layer]
        # compacted bytes: GPU rows == source rows at the GPU's own kept slots
        ri = np.arange(kept.shape[0])[:, None, None]
        hi = np.arange(kept.shape[1])[None, :, None]
        kk = np.arange(k_keep)[None, None, :]
        others = np.array(sorted(set(range(g.num_blocks)) - dst_blocks), dtype=np.int64)
        for pool_before, pool_after in ((case.k_pool[layer], run.k_pool[layer]),
                                        (case.v_pool[layer], run.v_pool[layer])):
            pb, pa = words(pool_before), words(pool_after)
            want = pb[ref.plan.src[ri, kept // b], hi, kept % b]        # [R][H][K_keep][W]
            got = pa[run.tables[ri, kk // b], hi, kk % b]
            bad = np.any(got != want, axis=-1)
            assert not bad.any(), f"layer {layer}: compacted rows differ at {np.argwhere(bad)[:5]}"
            # every block that is not a compaction target is untouched
            assert np.array_equal(pa[others], pb[others]), f"layer {layer}: a non-target block changed"
        if check_decode and run.out is not None:
            _check_decode(case, run, layer, stats)
    return stats


def _check_unit_scores_uniform(A, Rr, s, Ao, Ro, so, kept, ko, C, w, k_sel, layer, stats):
    """Scores and survivors when every request holds the same block count."""
    assert np.isfinite(A).all() and np.isfinite(Rr).all()
    okA = rel_ok(A, Ao, A_RTOL)
    assert okA.all(), f"layer {layer}: importance off at {np.argwhere(~okA)[:5]}"
    okR = np.abs(Rr - Ro) <= R_ATOL
    assert okR.all(), f"layer {layer}: redundancy off at {np.argwhere(~okR)[:5]}"
    okS = rel_ok(s[..., :C], so[..., :C], S_RTOL)
    assert okS.all(), f"layer {layer}: score off at {np.argwhere(~okS)[:5]}"
    stats["max_rel_A"] = max(stats["max_rel_A"], float(np.max(np.abs(A - Ao) / np.abs(Ao))))
    stats["max_abs_R"] = max(stats["max_abs_R"], float(np.max(np.abs(Rr - Ro))))
    stats["max_rel_s"] = max(stats["max_rel_s"],
                             float(np.max(np.abs(s[..., :C] - so[..., :C]) / np.abs(so[..., :C]))))
    # the GPU decision is exactly the selection rule applied to its own scores
    own = np.full(s.shape, np.nan)
    own[..., :C] = s[..., :C].astype(np.float64)
    np.testing.assert_array_equal(kept, oracle.select(own, w, k_sel))
    # and differs from the oracle's decision only at near-ties
    for r, h in zip(*np.nonzero(np.any(kept != ko, axis=-1))):
        gs, os_ = set(kept[r, h].tolist()), set(ko[r, h].tolist())
        tau = np.sort(so[r, h, :C])[::-1][k_sel - 1]
        for j in gs ^ os_:
            assert abs(so[r, h, j] - tau) <= TIE_RTOL * abs(tau), \
                f"layer {layer} req {r} head {h}: slot {j} differs, not a near tie"
        stats["near_tie_diffs"] += len(gs ^ os_)


def _check_ragged_unit_scores(A, Rr, s, Ao, Ro, so, kept, ko, Ts, w, k_sel, layer, stats):
    """Scores and survivors of requests holding different block counts: each
    request against the oracle on its own T; the debug rows past its T left
    as they were (NaN)."""
    for r, T in enumerate(Ts.tolist()):
        C = T - w
        a, rr, ss = A[r, :, :T], Rr[r, :, :T], s[r, :, :T]
        assert np.isnan(A[r, :, T:]).all() and np.isnan(s[r, :, T:]).all()
        assert np.isfinite(a).all() and np.isfinite(rr).all()
        okA = rel_ok(a, Ao[r, :, :T], A_RTOL)
        assert okA.all(), f"layer {layer} req {r}: importance off at {np.argwhere(~okA)[:5]}"
        okR = np.abs(rr - Ro[r, :, :T]) <= R_ATOL
        assert okR.all(), f"layer {layer} req {r}: redundancy off at {np.argwhere(~okR)[:5]}"
        okS = rel_ok(ss[:, :C], so[r, :, :C], S_RTOL)
        assert okS.all(), f"layer {layer} req {r}: score off at {np.argwhere(~okS)[:5]}"
        stats["max_rel_A"] = max(stats["max_rel_A"], float(np.max(np.abs(a - Ao[r, :, :T]) / np.abs(Ao[r, :, :T]))))
        stats["max_abs_R"] = max(stats["max_abs_R"], float(np.max(np.abs(rr - Ro[r, :, :T]))))
        own = np.full(ss.shape, np.nan)
        own[:, :C] = ss[:, :C].astype(np.float64)
        np.testing.assert_array_equal(kept[r], oracle.select(own, w, k_sel))
        for h in np.nonzero(np.any(kept[r] != ko[r], axis=-1))[0]:
            gs, os_ = set(kept[r, h].tolist()), set(ko[r, h].tolist())
            tau = np.sort(so[r, h, :C])[::-1][k_sel - 1]
            for j in gs ^ os_:
                assert abs(so[r, h, j] - tau) <= TIE_RTOL * abs(tau), \
                    f"layer {layer} req {r} head {h}: slot {j} differs, not a near tie"
            stats["near_tie_diffs"] += len(gs ^ os_)


def _check_decode(case, run, layer, stats):
    g = case.geom
    b, n_max = g.block_size, case.n_max
    k_keep = (n_max - 1) * b
    # oracle decode on the GPU-compacted, GPU-appended cache
    seq = np.full(run.tables.shape[0], k_keep + 1, dtype=np.int32)
    kp, vp = run.k_pool[layer].copy(), run.v_pool[layer].copy()
    slot = (run.tables[:, k_keep // b] * b + k_keep % b).astype(np.int32)
    oracle.append(kp, vp, case.k_new[layer], case.v_new[layer], slot)
    # run_case poisoned the reserved blocks' slots past the appended one
    res = run.tables[:, n_max - 1]
    kp[res, :, 1:, :] = run.appended_k[layer][res, :, 1:, :]
    vp[res, :, 1:, :] = run.appended_v[layer][res, :, 1:, :]
    assert np.array_equal(words(run.appended_k[layer]), words(kp))
    assert np.array_equal(words(run.appended_v[layer]), words(vp))
    want = oracle.decode(kp, vp, case.q_new[layer],
                         np.ascontiguousarray(run.tables[:, :n_max]), seq,
                         num_q_heads=g.num_q_heads)
    err = np.abs(run.out[layer] - want)
    assert np.isfinite(run.out[layer]).all()
    assert err.max() <= DECODE_ATOL, f"layer {layer}: decode error {err.max()}"
    stats["max_abs_out"] = max(stats["max_abs_out"], float(err.max()))
