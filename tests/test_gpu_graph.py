"""The allocation-free decode under HIP graph capture.

zp_paged_decode_noalloc exists for callers that cannot allocate, code under
graph capture among them.  A decode of a batch whose block lists are split
(the decode kernel and the split combine, partials in the fixed scratch) is
captured into a graph with torch; the graph is replayed several times, with
eager work and synchronisations between the replays and the query rewritten
in place before some of them, and every replay must equal, bit for bit, an
eager call on the same inputs (and the oracle, to the decode bar).
"""
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


@pytest.mark.parametrize("dtype,d,b,G,R,mb", [
    ("bf16", 128, 16, 4, 6, 128),   # split lists
    ("f32", 64, 32, 8, 5, 40),      # split, two query subgroups per KV head
])
def test_noalloc_decode_replays_from_a_graph(dtype, d, b, G, R, mb):
    import compressed_paged_kv_amd as zp
    from synth.device import to_tensor
    dev = "cuda"
    H = 2
    c = synth.make_case("graph", 7300 + d, num_reqs=R, num_layers=1, num_kv_heads=H,
                        num_q_heads=H * G, head_dim=d, block_size=b, n_max=mb, window=1,
                        num_blocks=R * mb + 2, dtype=dtype)
    say(f"[gpu graph] noalloc decode captured: R={R} H={H} G={G} d={d} b={b} "
        f"max_blocks={mb} {dtype}")
    rng = np.random.default_rng(7400 + d)
    seqs = rng.integers(1, mb * b + 1, size=R).astype(np.int32)
    cache = zp.KVCache([to_tensor(c.k_pool[0], dev)], [to_tensor(c.v_pool[0], dev)], H * G)
    assert zp.paged_decode_workspace_bytes(cache, R, mb) > 0, "the lists must be split"
    tab = torch.from_numpy(c.tables).to(dev)
    seq_t = torch.from_numpy(seqs).to(dev)
    q = to_tensor(c.q_new[0], dev)
    scale = 1.0 / np.sqrt(d)
    out = torch.zeros((R, H * G, d), dtype=torch.float32, device=dev)
    lse = torch.zeros((R, H * G), dtype=torch.float32, device=dev)
    # one eager call first: the fixed scratch's address is looked up outside the capture
    zp.paged_decode_noalloc(cache, 0, q, tab, seq_t, scale, out, lse_out=lse)
    torch.cuda.synchronize()

    def eager(q_now):
        o = torch.empty_like(out)
        l = torch.empty_like(lse)
        zp.paged_decode_noalloc(cache, 0, q_now, tab, seq_t, scale, o, lse_out=l)
        torch.cuda.synchronize()
        return o.cpu().numpy(), l.cpu().numpy()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            zp.paged_decode_noalloc(cache, 0, q, tab, seq_t, scale, out, lse_out=lse,
                                    stream=side)
    torch.cuda.synchronize()
    q_host = c.q_new[0].copy()
    for rep in range(4):
        if rep >= 2:  # a new query in the captured buffer
            q_host = q_host[::-1].copy()
            q.copy_(to_tensor(q_host, dev))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
        want, want_lse = eager(q)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
        np.testing.assert_array_equal(got_lse.view(np.uint32), want_lse.view(np.uint32))
        ref = oracle.decode(c.k_pool[0], c.v_pool[0], q_host, c.tables, seqs, num_q_heads=H * G)
        assert np.abs(got - ref).max() <= DECODE_ATOL, f"replay {rep}"
    say(f"[gpu graph] 4 replays equal the eager decode and the oracle")
