"""GPU parity of a stack of C4A layers under the IndexCache reuse schedule
(IndexCache freq2 page, section 2): layers the schedule marks as computing run
index top-k and attend with their own list; the others skip the indexer and
attend their own queries and pools with the list of the last computing layer.
Both sides follow the same schedule (taken from the library's host rule, which
the CPU tests pin to the oracle's) and are compared layer by layer."""
import numpy as np
import pytest

from helpers import (check_attention, check_topk_sets, gpu_attention, gpu_index_topk,
                     np_i32, oracle_attention, oracle_index_topk, to_device)
from sparse_long_context_compressor_amd import inputs as I

pytestmark = pytest.mark.gpu

RATIOS = [1, 4, 128, 4, 4, 128, 4, 4]


@pytest.fixture(scope="module")
def S():
    from sparse_long_context_compressor_amd import slc
    slc.lib()
    return slc


@pytest.mark.parametrize("freq,pattern", [(2, ""), (1, "FSSF")], ids=["freq2", "pattern"])
def test_reuse_chain_matches_oracle(S, oracle, freq, pattern):
    skips = S.indexcache_skips(RATIOS, freq, pattern)
    assert skips == oracle.indexcache_skips(RATIOS, freq, pattern)
    c4 = [i for i, r in enumerate(RATIOS) if r == 4]
    assert any(skips[i] for i in c4) and not skips[c4[0]]
    ctx, queries, n_slots = [3000, 1500], [(0, 2999), (1, 1499), (0, 2001)], [750, 375]
    ref_list = gpu_list = None
    for n, layer in enumerate(c4):
        lay = I.build_layer(40 + n, ratio=4, H=16, ctx=ctx, queries=queries, n_slots=n_slots,
                            W=128, k=128, H_I=16)
        computes = not skips[layer]
        if computes:
            ref_list, len_ref, sc_ref = oracle_index_topk(oracle, lay)
        out_ref, lse_ref = oracle_attention(oracle, lay, ref_list)
        to_device(lay)
        if computes:
            _, gpu_list, ln = gpu_index_topk(S, lay)
            nv = np.minimum((np_i32(lay.q_pos) + 1) // 4, np_i32(lay.n_slots)[np_i32(lay.q_seq)])
            check_topk_sets(gpu_list.cpu().numpy(), ln.cpu().numpy(), sc_ref, nv, lay.k)
            assert np.array_equal(ln.cpu().numpy(), len_ref)
        out, lse = gpu_attention(S, lay, gpu_list)
        check_attention(out, lse, out_ref, lse_ref)
        print(f"layer {layer}: {'compute' if computes else 'reuse'}", flush=True)
