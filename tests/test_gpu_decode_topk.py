"""slc_sparse_mla_decode_topk: the C4A top-k select and the decode over its
list in one call.  Its list, list length, output and lse must equal, bit for
bit, those of the two calls it stands for (slc_topk_select, then
slc_sparse_mla_decode over that list), which the other parity tests hold
against the oracle; the list is also checked against the exact top-k of the
scores and against the oracle's select, and at full size the attention is
checked against the oracle's.

Cases: the full 64K decode (bf16 and fp8 window pools); small layers whose
queries see fewer, exactly k and more than k slots (and none); score rows
built to drive each threshold path of the select (exact ties crowding the
threshold bin past the prefilter's candidate capacity, a crowded bin of
distinct keys, a bin of one key, -inf and signed zeros, k = 1 and k = n - 1);
shapes that take the two-launch form (rows longer than 16384 slots, a row
length that is not a multiple of 4, a split share above 512 entries)."""
import numpy as np
import pytest
import torch

from helpers import (check_attention, exact_topk_of, gpu_index_topk, np_i32, oracle_attention,
                     to_device)
from sparse_long_context_compressor_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    from sparse_long_context_compressor_amd import slc
    slc.lib()
    return slc


def nvis_of(lay):
    ns = np_i32(lay.n_slots)
    return np.minimum(ns[np_i32(lay.q_seq)], (np_i32(lay.q_pos) + 1) // 4).clip(0)


def two_step(S, lay, sc, ms, k):
    dev = lay.q.device
    idx = torch.empty((lay.n_q, k), dtype=torch.int32, device=dev)
    ln = torch.empty(lay.n_q, dtype=torch.int32, device=dev)
    S.topk_select(k, sc, ms, lay.q_seq, lay.q_pos, 4, lay.n_slots, idx, ln)
    out = torch.empty((lay.n_q, lay.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((lay.n_q, lay.H), dtype=torch.float32, device=dev)
    fl = S.SWA_FP8 if lay.swa_fp8 else 0
    S.sparse_mla_decode(4 | fl, lay.q, lay.q_seq, lay.q_pos, lay.W, lay.swa_pool, lay.swa_table,
                        lay.cmp_pool, lay.cmp_table, idx, lay.n_slots, lay.sm_scale, out, lse)
    return idx, ln, out, lse


def fused(S, lay, sc, ms, k):
    dev = lay.q.device
    idx = torch.full((lay.n_q, k), -7, dtype=torch.int32, device=dev)
    ln = torch.full((lay.n_q,), -7, dtype=torch.int32, device=dev)
    out = torch.full((lay.n_q, lay.H, 512), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((lay.n_q, lay.H), 7.0, dtype=torch.float32, device=dev)
    fl = S.SWA_FP8 if lay.swa_fp8 else 0
    S.sparse_mla_decode_topk(4 | fl, lay.q, lay.q_seq, lay.q_pos, lay.W, lay.swa_pool,
                             lay.swa_table, lay.cmp_pool, lay.cmp_table, k, sc, ms, lay.n_slots,
                             idx, ln, lay.sm_scale, out, lse)
    return idx, ln, out, lse


def assert_same(a, b, what):
    names = ("list", "length", "out", "lse")
    for x, y, n in zip(a, b, names):
        assert torch.equal(x, y), f"{what}: {n} differs from the two-call form"


@pytest.mark.parametrize("swa_fp8", [False, True], ids=["bf16_swa", "fp8_swa"])
def test_decode_topk_full_size(S, oracle, swa_fp8):
    lay = I.c4a_decode_64k(swa_fp8=swa_fp8)
    host = I.c4a_decode_64k(swa_fp8=swa_fp8)
    to_device(lay)
    sc, _, _ = gpu_index_topk(S, lay)
    ms = lay.max_slots
    ref = two_step(S, lay, sc, ms, lay.k)
    got = fused(S, lay, sc, ms, lay.k)
    torch.cuda.synchronize()
    assert_same(got, ref, "c4a_decode_64k")
    nv = nvis_of(host)
    idx = got[0].cpu().numpy()
    assert np.array_equal(idx, exact_topk_of(sc.cpu().numpy(), nv, lay.k))
    assert np.array_equal(got[1].cpu().numpy(), np.minimum(nv, lay.k))
    qs = np.array([0, 5, 13, 21, 31])
    out_ref, lse_ref = oracle_attention(oracle, host, idx[qs], queries=qs)
    kt = torch.as_tensor(qs, device=got[2].device)
    e = check_attention(got[2][kt], got[3][kt], out_ref, lse_ref)
    print(f"fused c4a_decode_64k (fp8 SWA {swa_fp8}): max abs {e[0]:.3g} rel L2 {e[1]:.3g} "
          f"lse {e[2]:.3g}")


# (H, W, k, queries, n_slots, ctx): queries of one or two sequences that see
# no slot, fewer than k, exactly k and more than k; H = 16 runs one head
# group per workgroup
SMALL = {
    "mixed_h64": (64, 128, 256, [(0, 2), (0, 1000), (0, 1023), (0, 1027), (0, 30000), (1, 8191),
                                 (1, 4000)], [7500, 2048], [30001, 8192]),
    "mixed_h16": (16, 64, 100, [(0, 399), (0, 403), (0, 9999), (1, 777)], [2500, 200],
                  [10000, 800]),
    "one_query_w0": (32, 0, 64, [(0, 16383)], [4096], [16384]),
}


@pytest.mark.parametrize("case", list(SMALL))
@pytest.mark.parametrize("swa_fp8", [False, True], ids=["bf16_swa", "fp8_swa"])
def test_decode_topk_small_layers(S, oracle, case, swa_fp8):
    H, W, k, queries, n_slots, ctx = SMALL[case]
    lay = I.build_layer(41, ratio=4, H=H, ctx=ctx, queries=queries, n_slots=n_slots, W=W, k=k,
                        H_I=16, swa_fp8=swa_fp8)
    host = I.build_layer(41, ratio=4, H=H, ctx=ctx, queries=queries, n_slots=n_slots, W=W, k=k,
                         H_I=16, swa_fp8=swa_fp8)
    to_device(lay)
    sc, _, _ = gpu_index_topk(S, lay)
    ms = lay.max_slots
    ref = two_step(S, lay, sc, ms, k)
    got = fused(S, lay, sc, ms, k)
    torch.cuda.synchronize()
    assert_same(got, ref, case)
    nv = nvis_of(host)
    idx = got[0].cpu().numpy()
    assert np.array_equal(idx, exact_topk_of(sc.cpu().numpy(), nv, k))
    out_ref, lse_ref = oracle_attention(oracle, host, idx)
    check_attention(got[2], got[3], out_ref, lse_ref)


def _rows():
    """(name, scores, k): one query that sees every slot of its row."""
    rng = np.random.default_rng(11)
    f32 = np.float32
    rows = []
    n = 16384
    v = rng.uniform(0.0, 0.74, n).astype(f32)
    ties = rng.choice(n, 2600, replace=False)
    v[ties[:300]] = rng.uniform(0.76, 1.0, 300).astype(f32)
    v[ties[300:]] = f32(0.75)          # 2300 equal keys: past the prefilter's 2048 candidates
    rows.append(("crowded_ties_16384", v, 512))
    n = 8192
    v = np.full(n, 1e-20, f32)
    pos = rng.permutation(n)
    v[pos[:300]] = f32(1e20)
    v[pos[300:1800]] = (np.float32(1.0).view(np.int32) + rng.permutation(1500)).astype(np.int32).view(f32)
    rows.append(("crowded_distinct_8192", v, 512))
    n = 4096
    v = (np.float32(1.0).view(np.int32) + rng.integers(0, 600, n)).astype(np.int32).view(f32)
    rows.append(("narrow_ties_4096", v, 100))
    n = 5000
    v = -rng.uniform(0.1, 10.0, n).astype(f32)
    pos = rng.permutation(n)
    v[pos[:1000]] = -np.inf
    v[pos[1000:1500]] = f32(-0.0)
    v[pos[1500:2000]] = f32(0.0)
    v[pos[2000:2300]] = rng.uniform(0.1, 5.0, 300).astype(f32)
    rows.append(("inf_and_signed_zeros_5000", v, 700))
    n = 12000
    v = rng.integers(0, 50, n).astype(f32)
    rows.append(("k1_with_ties_12000", v, 1))
    n = 1000
    v = rng.normal(size=n).astype(f32)
    rows.append(("k_n_minus_1_1000", v, 999))
    # full rows, where every wave of the select bounds the threshold by
    # itself: the top keys all in the first waves' slots (the other waves'
    # bounds sit far below them), heavy ties everywhere, and a row just long
    # enough for its last wave to hold k / 8 groups
    n = 16384
    v = rng.uniform(0.0, 1.0, n).astype(f32)
    v[rng.permutation(2000)[:600]] = (2.0 + rng.uniform(0.0, 1.0, 600)).astype(f32)
    rows.append(("wave_bound_concentrated_16384", v, 512))
    n = 16384
    v = rng.integers(0, 41, n).astype(f32)
    rows.append(("wave_bound_ties_16384", v, 512))
    n = 14592
    v = rng.normal(size=n).astype(f32)
    rows.append(("wave_bound_short_last_wave_14592", v, 512))
    # one query, k = 4096: 8 splits of exactly 512 list entries (the largest
    # share the one-launch form takes)
    n = 16384
    v = rng.normal(size=n).astype(f32)
    rows.append(("share_512_k4096", v, 4096))
    # the two-launch form: a row past 16384 slots, a row length not a
    # multiple of 4
    n = 20000
    v = rng.normal(size=n).astype(f32)
    rows.append(("two_launch_20000", v, 512))
    n = 777
    v = rng.normal(size=n).astype(f32)
    rows.append(("two_launch_777", v, 300))
    return rows


@pytest.mark.parametrize("name,row,k", _rows(), ids=[r[0] for r in _rows()])
def test_decode_topk_crafted_rows(S, oracle, name, row, k):
    n = row.shape[0]
    lay = I.build_layer(43, ratio=4, H=64, ctx=[4 * n], queries=[(0, 4 * n - 1)], n_slots=[n],
                        W=128, k=k, H_I=16)
    to_device(lay)
    sc = torch.from_numpy(row.reshape(1, n)).cuda()
    ref = two_step(S, lay, sc, n, k)
    got = fused(S, lay, sc, n, k)
    torch.cuda.synchronize()
    assert_same(got, ref, name)
    ref_idx, ref_len = oracle.topk(row, k)
    g = got[0].cpu().numpy()[0]
    assert int(got[1].item()) == ref_len == min(k, n)
    assert np.array_equal(g[:ref_len], np.sort(ref_idx[:ref_len])), name
    assert np.all(g[ref_len:] == -1)


def test_decode_topk_share_above_512(S, oracle):
    """32 queries x 64 heads at k = 4096: four splits of 1024 list entries, the
    two-launch form."""
    queries = [(b % 2, 32767 - 97 * b) for b in range(32)]
    lay = I.build_layer(45, ratio=4, H=64, ctx=[32768, 32768], queries=queries,
                        n_slots=[8192, 8192], W=128, k=4096, H_I=16)
    host = I.build_layer(45, ratio=4, H=64, ctx=[32768, 32768], queries=queries,
                         n_slots=[8192, 8192], W=128, k=4096, H_I=16)
    to_device(lay)
    sc, _, _ = gpu_index_topk(S, lay)
    ms = lay.max_slots
    ref = two_step(S, lay, sc, ms, lay.k)
    got = fused(S, lay, sc, ms, lay.k)
    torch.cuda.synchronize()
    assert_same(got, ref, "share_above_512")
    idx = got[0].cpu().numpy()
    assert np.array_equal(idx, exact_topk_of(sc.cpu().numpy(), nvis_of(host), lay.k))
    qs = np.array([0, 17, 31])
    out_ref, lse_ref = oracle_attention(oracle, host, idx[qs], queries=qs)
    kt = torch.as_tensor(qs, device=got[2].device)
    check_attention(got[2][kt], got[3][kt], out_ref, lse_ref)


def test_decode_topk_rejects_bad_arguments(S):
    lay = I.build_layer(44, ratio=4, H=16, ctx=[400], queries=[(0, 399)], n_slots=[100], W=16,
                        k=32, H_I=16)
    to_device(lay)
    sc = torch.zeros((1, 100), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, 32), dtype=torch.int32, device="cuda")
    ln = torch.empty(1, dtype=torch.int32, device="cuda")
    out = torch.empty((1, 16, 512), dtype=torch.bfloat16, device="cuda")
    for lt, k in ((128, 32), (1, 32), (4, 0), (4, 5000)):
        with pytest.raises(RuntimeError):
            S.sparse_mla_decode_topk(lt, lay.q, lay.q_seq, lay.q_pos, lay.W, lay.swa_pool,
                                     lay.swa_table, lay.cmp_pool, lay.cmp_table, k, sc, 100,
                                     lay.n_slots, idx, ln, lay.sm_scale, out, None)
