"""The allocation-free decode entry point (zp_paged_decode_noalloc) against
the decode that takes a caller workspace (zp_paged_decode_lse), through the
C ABI: output, log-sum-exp and recorded query bit-identical, on two calls in
a row -- the second with a smaller batch -- for a batch whose block lists
are split (partials in the fixed scratch) and one that is not; the outputs
also against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import DECODE_ATOL, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressed_paged_kv_amd as zp
    zp.lib()


def _batch(c, R, dev):
    from synth.device import to_tensor
    rng = np.random.default_rng(900 + R)
    b, mb = c.geom.block_size, c.tables.shape[1]
    seqs = rng.integers(0, mb * b + 1, size=R).astype(np.int32)
    seqs[0] = mb * b
    return (to_tensor(np.ascontiguousarray(c.q_new[0][:R]), dev),
            torch.from_numpy(np.ascontiguousarray(c.tables[:R])).to(dev),
            torch.from_numpy(seqs).to(dev), seqs)


@pytest.mark.parametrize("dtype,d,b,G,R1,R2,mb", [
    ("bf16", 128, 16, 4, 6, 3, 128),    # split lists (few requests, long lists)
    ("f32", 64, 32, 8, 5, 2, 40),       # split, G = 8 (two query subgroups)
    ("bf16", 128, 16, 4, 300, 200, 9),  # many requests: no split, scratch unused
])
def test_noalloc_decode_equals_workspace_decode_twice(dtype, d, b, G, R1, R2, mb):
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    H = 2
    c = synth.make_case("noalloc", 950 + R1, num_reqs=R1, num_layers=1, num_kv_heads=H,
                        num_q_heads=H * G, head_dim=d, block_size=b, n_max=mb, window=1,
                        num_blocks=R1 * mb + 3, dtype=dtype)
    say(f"[gpu noalloc] {dtype} d={d} b={b} G={G} max_blocks={mb}: calls of {R1} then {R2}")
    dev = "cuda"
    kp, vp = to_tensor(c.k_pool[0], dev), to_tensor(c.v_pool[0], dev)
    cache = zp.KVCache([kp], [vp], H * G)
    Hq = H * G
    for R in (R1, R2):
        q, tab, seq_t, seqs = _batch(c, R, dev)
        ws = torch.empty(max(zp.paged_decode_workspace_bytes(cache, R, mb), 16), dtype=torch.uint8,
                         device=dev)
        out_ws = torch.full((R, Hq, d), float("nan"), device=dev)
        lse_ws = torch.full((R, Hq), float("nan"), device=dev)
        qrec_ws = torch.full((R, Hq, d), float("nan"), dtype=q.dtype, device=dev)
        zp.paged_decode(cache, 0, q, tab, seq_t, 1.0 / np.sqrt(d), out_ws, ws, lse_out=lse_ws,
                        q_out=qrec_ws)
        out_na = torch.full((R, Hq, d), float("nan"), device=dev)
        lse_na = torch.full((R, Hq), float("nan"), device=dev)
        qrec_na = torch.full((R, Hq, d), float("nan"), dtype=q.dtype, device=dev)
        zp.paged_decode_noalloc(cache, 0, q, tab, seq_t, 1.0 / np.sqrt(d), out_na,
                                lse_out=lse_na, q_out=qrec_na)
        # and once more without the optional records
        out_na2 = torch.full((R, Hq, d), float("nan"), device=dev)
        zp.paged_decode_noalloc(cache, 0, q, tab, seq_t, 1.0 / np.sqrt(d), out_na2)
        torch.cuda.synchronize()
        a, bb, b2 = out_ws.cpu().numpy(), out_na.cpu().numpy(), out_na2.cpu().numpy()
        assert np.isfinite(bb).all()
        np.testing.assert_array_equal(a.view(np.uint32), bb.view(np.uint32))
        np.testing.assert_array_equal(a.view(np.uint32), b2.view(np.uint32))
        np.testing.assert_array_equal(lse_ws.cpu().numpy().view(np.uint32),
                                      lse_na.cpu().numpy().view(np.uint32))
        assert torch.equal(qrec_ws.view(torch.int16) if q.dtype == torch.bfloat16 else qrec_ws,
                           qrec_na.view(torch.int16) if q.dtype == torch.bfloat16 else qrec_na)
        want = oracle.decode(c.k_pool[0], c.v_pool[0], c.q_new[0][:R], c.tables[:R], seqs,
                             num_q_heads=Hq)
        assert np.abs(bb - want).max() <= DECODE_ATOL
        say(f"[gpu noalloc]   {R} requests (workspace {zp.paged_decode_workspace_bytes(cache, R, mb)} "
            f"bytes): bit-identical")
