"""The library's calls allocate nothing and never synchronise, so a whole
decode step can be captured in a HIP graph; every replay must reproduce the
eager result bit for bit, with unrelated eager work between replays."""
import pytest
import torch

from helpers import gpu_attention, gpu_index_topk, to_device
from sparse_long_context_compressor_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    from sparse_long_context_compressor_amd import slc
    lay = I.build_layer(21, ratio=4, H=64, ctx=[20000] * 4, queries=[(b, 19999) for b in range(4)],
                        n_slots=[5000] * 4, W=128, k=512, H_I=64)
    to_device(lay)
    dev = lay.q.device
    ms = lay.max_slots
    sc = torch.empty((lay.n_q, ms), dtype=torch.float32, device=dev)
    idx = torch.empty((lay.n_q, lay.k), dtype=torch.int32, device=dev)
    ln = torch.empty(lay.n_q, dtype=torch.int32, device=dev)
    out = torch.empty((lay.n_q, lay.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((lay.n_q, lay.H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(slc.sparse_mla_workspace_size(True, lay.n_q, lay.H, lay.W, lay.k), 256),
                     dtype=torch.uint8, device=dev)

    def step():
        slc.index_scores(lay.qi, lay.qi_scale, lay.qi_w, lay.q_seq, lay.q_pos, 4, lay.key_pool,
                         lay.key_table, lay.n_slots, ms, sc)
        slc.topk_select(lay.k, sc, ms, lay.q_seq, lay.q_pos, 4, lay.n_slots, idx, ln)
        slc.sparse_mla_decode(4, lay.q, lay.q_seq, lay.q_pos, lay.W, lay.swa_pool, lay.swa_table,
                              lay.cmp_pool, lay.cmp_table, idx, lay.n_slots, lay.sm_scale, out,
                              lse, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, ln, out.view(torch.int16), lse)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        for t in (idx, ln, out, lse):
            t.zero_()
        junk = torch.randn(1 << 20, device=dev).sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (idx, ln, out.view(torch.int16), lse)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {r} differs"
        assert torch.isfinite(junk)
