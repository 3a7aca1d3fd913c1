"""The no-allocation decode (slc_sparse_mla_decode_noalloc, split partials in
the library's static device array) against the decode with a caller
workspace, through the C ABI: bit-identical outputs and lse on two calls in a
row, the second with a smaller input (so stale partials of the first call in
the shared array must not leak into the second)."""
import numpy as np
import pytest
import torch

from sparse_long_context_compressor_amd import inputs as I
from sparse_long_context_compressor_amd import slc as S

pytestmark = pytest.mark.gpu


def _both(lay, idx):
    dev = lay.q.device
    outs = []
    for noalloc in (False, True):
        out = torch.full((lay.n_q, lay.H, 512), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((lay.n_q, lay.H), float("nan"), dtype=torch.float32, device=dev)
        f = S.sparse_mla_decode_noalloc if noalloc else S.sparse_mla_decode
        f(lay.ratio, lay.q, lay.q_seq, lay.q_pos, lay.W, lay.swa_pool, lay.swa_table,
          lay.cmp_pool, lay.cmp_table, idx, lay.n_slots, sm_scale=lay.sm_scale, out=out, lse=lse)
        outs.append((out, lse))
    torch.cuda.synchronize()
    return outs


def test_noalloc_decode_equals_workspace_decode_twice():
    S.lib()
    big = I.c4a_decode_64k(seed=9, device="cuda")
    need = S.sparse_mla_workspace_size(True, big.n_q, big.H, big.W, big.k)
    assert 0 < need <= S.sparse_mla_decode_noalloc_max_bytes()
    g = torch.Generator().manual_seed(3)
    idx = torch.stack([torch.randperm(16384, generator=g)[:512] for _ in range(big.n_q)]).to(
        torch.int32).cuda()
    (o1, l1), (o2, l2) = _both(big, idx)
    assert torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # a smaller call right after: fewer queries and heads, another window and list
    small = I.build_layer(10, ratio=4, H=32, ctx=[3000, 900, 5000],
                          queries=[(0, 2999), (1, 899), (2, 4999)], n_slots=[750, 225, 1250],
                          W=96, k=200, given_topk=True, device="cuda")
    assert 0 < S.sparse_mla_workspace_size(True, small.n_q, small.H, small.W, small.k) < need
    (o1, l1), (o2, l2) = _both(small, small.given_idx)
    assert torch.isfinite(l1).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_decode_rejects_shapes_beyond_its_array():
    S.lib()
    lay = I.build_layer(11, ratio=4, H=16, ctx=[600], queries=[(0, 599)], n_slots=[150], W=16,
                        k=32, given_topk=True, device="cuda")
    n_q = 100           # 100 queries x 64 heads in two splits: 13 MB of partials
    assert S.sparse_mla_workspace_size(True, n_q, 64, 128, 512) > \
        S.sparse_mla_decode_noalloc_max_bytes()
    q = torch.zeros((n_q, 64, 576), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    idx = torch.zeros((n_q, 512), dtype=torch.int32, device="cuda")
    out = torch.zeros((n_q, 64, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(S.SlcError) as e:
        S.sparse_mla_decode_noalloc(4, q, z, z, 128, lay.swa_pool, lay.swa_table, lay.cmp_pool,
                                    lay.cmp_table, idx, lay.n_slots, 0.1, out, None)
    assert e.value.status == S.SLC_ERR_WORKSPACE
    assert not out.any()
