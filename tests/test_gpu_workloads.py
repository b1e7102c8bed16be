"""GPU parity of the wider workloads at their full sizes, and of compression
overlapped with decode on a second stream.

The full-size caches (up to 8.6 GB per layer) are generated on the device
(``synth.device_gen``); the oracle then reruns sampled (layer, request)
units from the bytes copied back to the host, before and after the call:
importance, redundancy and score within tolerance, the GPU survivor set equal
to the selection rule on the GPU's own scores and to the oracle's up to
near-ties, compacted rows bit-exact, and the decode output of the sampled
requests within 2e-3.  The target plan, refcounts and freed ids are compared
exactly for the whole batch (host integers only).
"""
import numpy as np
import pytest
import torch

import compressed_paged_kv_amd as zp
import oracle
import synth
from gpu_common import A_RTOL, DECODE_ATOL, R_ATOL, S_RTOL, TIE_RTOL, rel_ok, say, words
from synth.device import to_numpy, to_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zp.lib()  # raises if the HIP library is missing


def _blocks(pool_t, ids) -> np.ndarray:
    idx = torch.from_numpy(np.asarray(ids, dtype=np.int64)).to(pool_t.device)
    return to_numpy(pool_t.index_select(0, idx))


def _check_unit_scores(A, Rr, s, Ao, Ro, so, C, tag):
    okA = rel_ok(A, Ao, A_RTOL)
    assert okA.all(), f"{tag}: importance off at {np.argwhere(~okA)[:5]}"
    okR = np.abs(Rr - Ro) <= R_ATOL
    assert okR.all(), f"{tag}: redundancy off at {np.argwhere(~okR)[:5]}"
    okS = rel_ok(s[..., :C], so[..., :C], S_RTOL)
    assert okS.all(), f"{tag}: score off at {np.argwhere(~okS)[:5]}"


def _check_unit_kept(kept, s, so, w, k_sel, C, tag):
    own = np.full(s.shape, np.nan)
    own[..., :C] = s[..., :C].astype(np.float64)
    np.testing.assert_array_equal(kept, oracle.select(own, w, k_sel))
    ko = oracle.select(so, w, k_sel)
    for h in np.nonzero(np.any(kept != ko, axis=-1))[0]:
        tau = np.sort(so[h, :C])[::-1][k_sel - 1]
        for j in set(kept[h].tolist()) ^ set(ko[h].tolist()):
            assert abs(so[h, j] - tau) <= TIE_RTOL * abs(tau), f"{tag} head {h}: slot {j} not a near tie"


def _run_sampled(case, samples, label):
    """Compress the whole device case, append the pending token, decode;
    check the sampled (layer, request) units against the oracle."""
    dev = case.k_pool[0].device
    g = case.geom
    L, H, Hq, d, b = g.num_layers, g.num_kv_heads, g.num_q_heads, g.head_dim, g.block_size
    n_max, w = case.n_max, case.window
    R = case.num_reqs
    T, k_keep = n_max * b, (n_max - 1) * b
    C, k_sel = T - w, k_keep - w
    # snapshots of the sampled units' source blocks (logical order)
    snap = {(l, r): (_blocks(case.k_pool[l], case.tables[r]), _blocks(case.v_pool[l], case.tables[r]))
            for l, r in samples}
    prefix = None
    if g.num_blocks and (case.refcounts > 1).any():
        shared = np.nonzero(case.refcounts > 1)[0]
        prefix = {l: (_blocks(case.k_pool[l], shared), _blocks(case.v_pool[l], shared))
                  for l in sorted({l for l, _ in samples})}
    cache = zp.KVCache(case.k_pool, case.v_pool, Hq)
    pool = zp.BlockPool.from_refcounts(case.refcounts)
    tables = case.tables.copy()
    ws = torch.empty(zp.compress_workspace_bytes(cache, R, n_max, w), dtype=torch.uint8, device=dev)
    dbg = dict(importance=torch.full((L, R, H, T), float("nan"), device=dev),
               redundancy=torch.full((L, R, H, T), float("nan"), device=dev),
               score=torch.full((L, R, H, T), float("nan"), device=dev),
               kept=torch.full((L, R, H, k_keep), -1, dtype=torch.int32, device=dev))
    say(f"{label}: compress {L} layer(s) x {R} requests, T={T}, rows={g.group * w}")
    freed = zp.compress(cache, pool, n_max, w, tables, case.window_q, ws, debug=dbg)
    torch.cuda.synchronize()
    # bookkeeping, exact, for the whole batch
    ref = oracle.plan(case.refcounts, case.tables, n_max)
    assert ref.status == oracle.OK
    np.testing.assert_array_equal(tables, ref.tables)
    pool.sync()
    np.testing.assert_array_equal(pool.refcounts(), ref.refcounts)
    np.testing.assert_array_equal(np.sort(freed), np.sort(ref.freed))
    # append + decode every layer
    slot = tables[:, k_keep // b] * b + k_keep % b
    slot_t = torch.from_numpy(slot.astype(np.int32)).to(dev)
    tab_t = torch.from_numpy(tables).to(dev)
    seq = torch.full((R,), k_keep + 1, dtype=torch.int32, device=dev)
    dws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, n_max), 16), dtype=torch.uint8,
                      device=dev)
    outs = {}
    compacted = {}
    for l in sorted({l for l, _ in samples}):
        for r in sorted({r for ll, r in samples if ll == l}):
            compacted[(l, r)] = (_blocks(case.k_pool[l], tables[r]), _blocks(case.v_pool[l], tables[r]))
    say(f"{label}: append + decode")
    for l in range(L):
        zp.append_kv(cache, l, case.k_new[l], case.v_new[l], slot_t)
        out = torch.empty((R, Hq, d), dtype=torch.float32, device=dev)
        zp.paged_decode(cache, l, case.q_new[l], tab_t, seq, 1.0 / np.sqrt(d), out, dws)
        if any(ll == l for ll, _ in samples):
            outs[l] = out
    torch.cuda.synchronize()
    A_all = dbg["importance"]
    near = 0
    for l, r in samples:
        tag = f"{label} layer {l} req {r}"
        say(f"  oracle on {tag}")
        kb, vb = snap[(l, r)]
        src = np.arange(n_max, dtype=np.int32)[None, :]
        wq = to_numpy(case.window_q[l][r:r + 1])
        Ao, Ro, so = oracle.scores(kb, wq, src, num_kv_heads=H, num_q_heads=Hq, head_dim=d,
                                   block_size=b, n_max=n_max, window=w)
        A = A_all[l, r].cpu().numpy()
        Rr = dbg["redundancy"][l, r].cpu().numpy()
        s = dbg["score"][l, r].cpu().numpy()
        _check_unit_scores(A, Rr, s, Ao[0], Ro[0], so[0], C, tag)
        kept = dbg["kept"][l, r].cpu().numpy()
        _check_unit_kept(kept, s, so[0], w, k_sel, C, tag)
        near += int(np.count_nonzero(kept != oracle.select(so[0], w, k_sel)))
        # compacted rows: GPU target rows == source rows at the GPU's kept slots
        ck, cv = compacted[(l, r)]
        hi = np.arange(H)[:, None]
        kk = np.arange(k_keep)[None, :]
        for before, after in ((kb, ck), (vb, cv)):
            want = words(before)[kept // b, hi, kept % b]
            got = words(after)[kk // b, hi, kk % b]
            assert np.array_equal(got, want), f"{tag}: compacted rows differ"
        # decode of this request on the GPU-compacted cache plus the appended token
        kp, vp = ck.copy(), cv.copy()
        oracle.append(kp, vp, to_numpy(case.k_new[l][r:r + 1]), to_numpy(case.v_new[l][r:r + 1]),
                      np.array([(k_keep // b) * b + k_keep % b], dtype=np.int32))
        want = oracle.decode(kp, vp, to_numpy(case.q_new[l][r:r + 1]), src,
                             np.array([k_keep + 1], dtype=np.int32), num_q_heads=Hq)
        got = outs[l][r:r + 1].cpu().numpy()
        err = float(np.abs(got - want).max())
        assert np.isfinite(got).all() and err <= DECODE_ATOL, f"{tag}: decode error {err}"
    if prefix is not None:
        shared = np.nonzero(case.refcounts > 1)[0]
        for l, (kb, vb) in prefix.items():
            assert np.array_equal(words(_blocks(case.k_pool[l], shared)), words(kb)), "prefix K changed"
            assert np.array_equal(words(_blocks(case.v_pool[l], shared)), words(vb)), "prefix V changed"
    say(f"{label}: ok ({len(samples)} sampled units, {near} near-tie slot differences)")
    pool.close()


def test_structured_b32_full_size_sampled():
    """512 requests, budget 4096 (b=32, w=32, 128 window rows), AR(1) keys with
    planted large keys: the two-row-group scoring path at its largest T."""
    from synth.device_gen import case_structured_device
    say("structured_b32_budget4096: generating on the device")
    case = case_structured_device(torch.device("cuda:0"))
    _run_sampled(case, [(0, 0), (0, 137), (0, 311), (0, 511)], "structured_b32_budget4096")


def test_shared_prefix_full_size_sampled():
    """32 requests x 32 layers sharing a 32-block prefix: 1024 new targets,
    the 32 prefix blocks freed, prefix bytes unchanged."""
    from synth.device_gen import case_shared_prefix_device
    say("shared_prefix_32req_32layers: generating on the device")
    case = case_shared_prefix_device(torch.device("cuda:0"))
    _run_sampled(case, [(0, 0), (17, 13), (31, 31)], "shared_prefix_32req_32layers")


def test_compress_overlapped_with_decode():
    """Compression of two requests on one stream while the others append and
    decode on another (the decode of the next step waiting on an event); all
    eight requests share a 4-block prefix, which the compression re-targets
    while the decode reads it: results bit-identical to running the same
    work serially, the shared blocks unchanged, and equal to the oracle."""
    say("overlap: 8 requests x 3 layers sharing 4 blocks, 2 compress on stream A, 6 decode on B")
    dev = torch.device("cuda:0")
    P = 4
    base = synth.make_case("overlap", 301, num_reqs=8, num_layers=3, num_kv_heads=2, num_q_heads=8,
                           head_dim=128, block_size=16, n_max=24, window=16, num_blocks=256,
                           dtype="bf16", key_scale_range=(0.5, 2.0), shared_prefix_blocks=P)
    g = base.geom
    L, H, Hq, d, b = g.num_layers, g.num_kv_heads, g.num_q_heads, g.head_dim, g.block_size
    n_max, w = base.n_max, base.window
    T, k_keep = n_max * b, (n_max - 1) * b
    comp, dec = np.array([1, 5]), np.array([0, 2, 3, 4, 6, 7])
    rng = np.random.default_rng(3011)
    # appends land past the shared prefix (a shared block is never written)
    lens = rng.integers(P * b, T - 1, size=len(dec)).astype(np.int32)
    lens[0] = T - 1                      # a full last block but for the appended slot
    tables_c = np.ascontiguousarray(base.tables[comp])
    tables_d = np.ascontiguousarray(base.tables[dec])
    slot_d = (tables_d[np.arange(len(dec)), lens // b] * b + lens % b).astype(np.int32)

    def run(overlap: bool):
        kp = [to_tensor(x, dev) for x in base.k_pool]
        vp = [to_tensor(x, dev) for x in base.v_pool]
        cache = zp.KVCache(kp, vp, Hq)
        pool = zp.BlockPool.from_refcounts(base.refcounts)
        tabc = tables_c.copy()
        wq = [to_tensor(np.ascontiguousarray(x[comp]), dev) for x in base.window_q]
        qd = [to_tensor(np.ascontiguousarray(x[dec]), dev) for x in base.q_new]
        kd = [to_tensor(np.ascontiguousarray(x[dec]), dev) for x in base.k_new]
        vd = [to_tensor(np.ascontiguousarray(x[dec]), dev) for x in base.v_new]
        ws = torch.empty(zp.compress_workspace_bytes(cache, len(comp), n_max, w), dtype=torch.uint8,
                         device=dev)
        dws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, len(dec), n_max), 16),
                          dtype=torch.uint8, device=dev)
        tab_t = torch.from_numpy(tables_d).to(dev)
        slot_t = torch.from_numpy(slot_d).to(dev)
        seq_t = torch.from_numpy(lens + 1).to(dev)
        kept = torch.full((L, len(comp), H, k_keep), -1, dtype=torch.int32, device=dev)
        outs = [torch.empty((len(dec), Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        if overlap:
            ev = torch.cuda.Event()
            ev.record(sb)            # stream B: the previous step's decode is done
            sa.wait_event(ev)
            zp.compress(cache, pool, n_max, w, tabc, wq, ws, stream=sa, debug={"kept": kept})
            for l in range(L):
                zp.append_kv(cache, l, kd[l], vd[l], slot_t, stream=sb)
                zp.paged_decode(cache, l, qd[l], tab_t, seq_t, 1.0 / np.sqrt(d), outs[l], dws,
                                stream=sb)
        else:
            zp.compress(cache, pool, n_max, w, tabc, wq, ws, stream=sa, debug={"kept": kept})
            sa.synchronize()
            for l in range(L):
                zp.append_kv(cache, l, kd[l], vd[l], slot_t, stream=sa)
                zp.paged_decode(cache, l, qd[l], tab_t, seq_t, 1.0 / np.sqrt(d), outs[l], dws,
                                stream=sa)
        torch.cuda.synchronize()
        pool.sync()
        return (tabc, kept.cpu().numpy(), [to_numpy(t) for t in kp], [to_numpy(t) for t in vp],
                np.stack([o.cpu().numpy() for o in outs]))

    ser = run(False)
    say("overlap: serial run done")
    ovl = run(True)
    say("overlap: overlapped run done")
    np.testing.assert_array_equal(ser[0], ovl[0])
    np.testing.assert_array_equal(ser[1], ovl[1])
    for l in range(L):
        assert np.array_equal(words(ser[2][l]), words(ovl[2][l]))
        assert np.array_equal(words(ser[3][l]), words(ovl[3][l]))
    np.testing.assert_array_equal(ser[4].view(np.uint32), ovl[4].view(np.uint32))
    shared = base.tables[0, :P]
    assert np.all(base.tables[:, :P] == shared)
    assert not np.any(np.isin(ovl[0], shared))        # the compressed requests left the prefix
    for l in range(L):                                 # ... and never wrote it
        assert np.array_equal(words(ovl[2][l][shared]), words(base.k_pool[l][shared]))
        assert np.array_equal(words(ovl[3][l][shared]), words(base.v_pool[l][shared]))
    # the compressing requests against the oracle (their own sub-batch)
    sub = synth.CompressCase("overlap_comp", base.seed, g, n_max, w, tables_c,
                             np.bincount(tables_c.reshape(-1), minlength=g.num_blocks).astype(np.int32),
                             base.k_pool, base.v_pool, [x[comp] for x in base.window_q],
                             [x[comp] for x in base.q_new], [x[comp] for x in base.k_new],
                             [x[comp] for x in base.v_new])
    ref = oracle.compress(sub, with_pools=False)
    for l in range(L):
        ko = ref.kept[l]
        diff = np.nonzero(np.any(ovl[1][l] != ko, axis=-1))
        for r, h in zip(*diff):
            so = ref.s[l][r, h]
            tau = np.sort(so[:T - w])[::-1][k_keep - w - 1]
            for j in set(ovl[1][l][r, h].tolist()) ^ set(ko[r, h].tolist()):
                assert abs(so[j] - tau) <= TIE_RTOL * abs(tau)
    # the decoding requests against the oracle (append + dense decode)
    for l in range(L):
        kp, vp = base.k_pool[l].copy(), base.v_pool[l].copy()
        oracle.append(kp, vp, base.k_new[l][dec], base.v_new[l][dec], slot_d)
        want = oracle.decode(kp, vp, base.q_new[l][dec], tables_d, lens + 1, num_q_heads=Hq)
        err = float(np.abs(ovl[4][l] - want).max())
        assert err <= DECODE_ATOL, f"layer {l}: decode error {err}"
    say("overlap: ok")


def _poison_past(pool_t, tables, upto, b):
    """NaN into every slot at or past logical slot upto[r] of each request
    (whole blocks past it, and the tail of the block it falls in): a decode
    that read past a request's length would turn its output NaN."""
    full = [tables[r, (int(upto[r]) + b - 1) // b:] for r in range(tables.shape[0])]
    ids = np.concatenate(full) if full else np.zeros(0, np.int32)
    if ids.size:
        pool_t.index_fill_(0, torch.from_numpy(ids.astype(np.int64)).to(pool_t.device),
                           float("nan"))
    part = {}
    for r in range(tables.shape[0]):
        o = int(upto[r]) % b
        if o:
            part.setdefault(o, []).append(int(tables[r, int(upto[r]) // b]))
    for o, lst in part.items():
        idx = torch.tensor(lst, dtype=torch.int64, device=pool_t.device)
        pool_t[idx, :, o:, :] = float("nan")


def test_mix_full_size_two_streams_sampled():
    """The continuous-batching mix at its full size: 256 requests x 36 layers
    of the Qwen3-8B shape (pool 32768 blocks, 72 GiB of K/V).  A seeded 10 %
    of the requests (26) sit at the cap and compress on one stream while the
    other 230, with ragged cached lengths in [64, 2048), append one token and
    decode in every layer on a second stream, the two joined by events; then
    the compressed requests rejoin decoding (append at slot 2032, decode over
    2033).  The plan, refcounts and freed ids are compared exactly for the
    whole batch; sampled (layer, request) compressions -- scores, survivor
    sets, compacted rows -- and sampled decodes of both groups against the
    oracle.  Slots past every decoding request's length are NaN, so a decode
    reading past it would fail."""
    from synth.device_gen import case_mix_device
    dev = torch.device("cuda:0")
    say("mix_qwen3_8b_36layers: generating 256 requests x 36 layers on the device")
    case = case_mix_device(dev)
    g = case.geom
    L, H, Hq, d, b = g.num_layers, g.num_kv_heads, g.num_q_heads, g.head_dim, g.block_size
    n_max, w = case.n_max, case.window
    T, k_keep = n_max * b, (n_max - 1) * b
    C, k_sel = T - w, k_keep - w
    lens = case.seq_lens
    comp = np.nonzero(lens == T)[0]
    dec = np.nonzero(lens < T)[0]
    Rc, Rd = len(comp), len(dec)
    assert Rc == 26 and Rd == 230, (Rc, Rd)
    tables_c = np.ascontiguousarray(case.tables[comp])
    tables_d = np.ascontiguousarray(case.tables[dec])
    ld = lens[dec].astype(np.int32)
    say(f"mix: poisoning slots past the {Rd} decoding requests' lengths")
    for l in range(L):
        for t in (case.k_pool[l], case.v_pool[l]):
            _poison_past(t, tables_d, ld + 1, b)
    comp_t = torch.from_numpy(comp.astype(np.int64)).to(dev)
    dec_t = torch.from_numpy(dec.astype(np.int64)).to(dev)
    wq = [q.index_select(0, comp_t).contiguous() for q in case.window_q]
    qd = [q.index_select(0, dec_t).contiguous() for q in case.q_new]
    kd = [k.index_select(0, dec_t).contiguous() for k in case.k_new]
    vd = [v.index_select(0, dec_t).contiguous() for v in case.v_new]
    qc = [q.index_select(0, comp_t).contiguous() for q in case.q_new]
    kc = [k.index_select(0, comp_t).contiguous() for k in case.k_new]
    vc = [v.index_select(0, comp_t).contiguous() for v in case.v_new]

    c_samples = [(0, 0), (11, 7), (23, 13), (35, 25)]           # (layer, index into comp)
    order = np.argsort(ld)
    d_samples = [(0, int(order[0])), (7, int(order[-1])), (18, int(order[len(order) // 2])),
                 (35, 101), (29, 3)]                             # (layer, index into dec)
    snap_c = {(l, i): (_blocks(case.k_pool[l], tables_c[i]), _blocks(case.v_pool[l], tables_c[i]))
              for l, i in c_samples}
    snap_d = {(l, i): (_blocks(case.k_pool[l], tables_d[i]), _blocks(case.v_pool[l], tables_d[i]))
              for l, i in d_samples}

    cache = zp.KVCache(case.k_pool, case.v_pool, Hq)
    pool = zp.BlockPool.from_refcounts(case.refcounts)
    tables = tables_c.copy()
    ws = torch.empty(zp.compress_workspace_bytes(cache, Rc, n_max, w), dtype=torch.uint8, device=dev)
    # one workspace for both decodes on stream B (the 26 rejoining requests
    # split their block lists, the 230 others do not)
    dws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, Rd, n_max),
                          zp.paged_decode_workspace_bytes(cache, Rc, n_max), 16),
                      dtype=torch.uint8, device=dev)
    dbg = dict(importance=torch.full((L, Rc, H, T), float("nan"), device=dev),
               redundancy=torch.full((L, Rc, H, T), float("nan"), device=dev),
               score=torch.full((L, Rc, H, T), float("nan"), device=dev),
               kept=torch.full((L, Rc, H, k_keep), -1, dtype=torch.int32, device=dev))
    tab_d = torch.from_numpy(tables_d).to(dev)
    slot_d = torch.from_numpy((tables_d[np.arange(Rd), ld // b] * b + ld % b).astype(np.int32)).to(dev)
    seq_d = torch.from_numpy(ld + 1).to(dev)
    out_d = torch.full((L, Rd, Hq, d), float("nan"), device=dev)
    s_c, s_d = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    say(f"mix: {Rc} requests compress 36 layers on stream A, {Rd} append + decode on stream B")
    start = torch.cuda.Event()
    start.record(torch.cuda.current_stream())
    s_c.wait_event(start)
    s_d.wait_event(start)
    freed = zp.compress(cache, pool, n_max, w, tables, wq, ws, stream=s_c, debug=dbg)
    for l in range(L):
        zp.append_kv(cache, l, kd[l], vd[l], slot_d, stream=s_d)
        zp.paged_decode(cache, l, qd[l], tab_d, seq_d, 1.0 / np.sqrt(d), out_d[l], dws, stream=s_d)
    done_c = torch.cuda.Event()
    done_c.record(s_c)
    # the compressed requests rejoin decoding after the compression
    s_d.wait_event(done_c)
    tab_c_t = torch.from_numpy(np.ascontiguousarray(tables)).to(dev)
    slot_c = torch.from_numpy((tables[:, k_keep // b] * b + k_keep % b).astype(np.int32)).to(dev)
    seq_c = torch.full((Rc,), k_keep + 1, dtype=torch.int32, device=dev)
    out_c = torch.full((L, Rc, Hq, d), float("nan"), device=dev)
    for l in range(L):
        zp.append_kv(cache, l, kc[l], vc[l], slot_c, stream=s_d)
        zp.paged_decode(cache, l, qc[l], tab_c_t, seq_c, 1.0 / np.sqrt(d), out_c[l], dws, stream=s_d)
    torch.cuda.synchronize()
    say("mix: checking the plan of the whole batch")
    ref = oracle.plan(case.refcounts[:], tables_c, n_max)
    assert ref.status == oracle.OK
    np.testing.assert_array_equal(tables, ref.tables)
    pool.sync()
    # the decoding requests still hold their blocks: the pool counts every table
    np.testing.assert_array_equal(pool.refcounts(), ref.refcounts)
    np.testing.assert_array_equal(np.sort(freed), np.sort(ref.freed))
    assert np.isfinite(out_d.cpu().numpy()).all() and np.isfinite(out_c.cpu().numpy()).all()
    near = 0
    for l, i in c_samples:
        tag = f"mix compress layer {l} req {int(comp[i])}"
        say(f"  oracle on {tag}")
        kb, vb = snap_c[(l, i)]
        src = np.arange(n_max, dtype=np.int32)[None, :]
        Ao, Ro, so = oracle.scores(kb, to_numpy(wq[l][i:i + 1]), src, num_kv_heads=H,
                                   num_q_heads=Hq, head_dim=d, block_size=b, n_max=n_max, window=w)
        A = dbg["importance"][l, i].cpu().numpy()
        Rr = dbg["redundancy"][l, i].cpu().numpy()
        s = dbg["score"][l, i].cpu().numpy()
        _check_unit_scores(A, Rr, s, Ao[0], Ro[0], so[0], C, tag)
        kept = dbg["kept"][l, i].cpu().numpy()
        _check_unit_kept(kept, s, so[0], w, k_sel, C, tag)
        near += int(np.count_nonzero(kept != oracle.select(so[0], w, k_sel)))
        ck, cv = _blocks(case.k_pool[l], tables[i]), _blocks(case.v_pool[l], tables[i])
        hi = np.arange(H)[:, None]
        kk = np.arange(k_keep)[None, :]
        for before, after in ((kb, ck), (vb, cv)):
            want = words(before)[kept // b, hi, kept % b]
            got = words(after)[kk // b, hi, kk % b]
            assert np.array_equal(got, want), f"{tag}: compacted rows differ"
        # the rejoining decode: compacted rows + the token appended at slot
        # k_keep (offset 0 of the reserved block), which must be bit-exact
        kp, vp = ck.copy(), cv.copy()
        oracle.append(kp, vp, to_numpy(kc[l][i:i + 1]), to_numpy(vc[l][i:i + 1]),
                      np.array([k_keep], dtype=np.int32))
        assert np.array_equal(words(kp), words(ck)) and np.array_equal(words(vp), words(cv)), \
            f"{tag}: rejoining append"
        want = oracle.decode(kp, vp, to_numpy(qc[l][i:i + 1]), src,
                             np.array([k_keep + 1], dtype=np.int32), num_q_heads=Hq)
        err = float(np.abs(out_c[l, i:i + 1].cpu().numpy() - want).max())
        assert err <= DECODE_ATOL, f"{tag}: rejoining decode error {err}"
    for l, i in d_samples:
        tag = f"mix decode layer {l} req {int(dec[i])} (len {int(ld[i])})"
        say(f"  oracle on {tag}")
        kb, vb = snap_d[(l, i)]
        src = np.arange(n_max, dtype=np.int32)[None, :]
        kp, vp = kb.copy(), vb.copy()
        oracle.append(kp, vp, to_numpy(kd[l][i:i + 1]), to_numpy(vd[l][i:i + 1]),
                      np.array([int(ld[i])], dtype=np.int32))
        after_k, after_v = _blocks(case.k_pool[l], tables_d[i]), _blocks(case.v_pool[l], tables_d[i])
        assert np.array_equal(words(after_k), words(kp)), f"{tag}: append wrote elsewhere"
        assert np.array_equal(words(after_v), words(vp)), f"{tag}: append wrote elsewhere"
        want = oracle.decode(kp, vp, to_numpy(qd[l][i:i + 1]), src,
                             np.array([int(ld[i]) + 1], dtype=np.int32), num_q_heads=Hq)
        err = float(np.abs(out_d[l, i:i + 1].cpu().numpy() - want).max())
        assert err <= DECODE_ATOL, f"{tag}: decode error {err}"
    say(f"mix: ok ({len(c_samples)} compressions, {len(c_samples) + len(d_samples)} decodes "
        f"sampled, {near} near-tie slot differences)")
    pool.close()
