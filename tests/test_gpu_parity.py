"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs,
at sizes the oracle finishes in seconds (several tiles, ragged tails, edge
cases).  Acceptance rules as stated in each test."""
import numpy as np
import pytest
import torch

from helpers import (POOL_FP32_REL, bits16, check_attention, check_topk_sets, exact_topk_of,
                     fp8_values, gpu_attention, gpu_index_topk, near_bf16_midpoint_within,
                     near_midpoint_within, near_scale_boundary, np_f32, np_i32, np_u8, oracle_attention,
                     oracle_compress, oracle_index_topk, pool_magnitude, to_device)
from sparse_long_context_compressor_amd import inputs as I
from sparse_long_context_compressor_amd import pools as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    from sparse_long_context_compressor_amd import slc
    slc.lib()
    return slc


def pow2_rule(amax: np.ndarray) -> np.ndarray:
    """Per block: the smallest 2^e with amax <= 448 * 2^e, e >= -126 (1 for
    amax = 0).  With amax = f * 2^x, f in [0.5, 1), and 448 = 0.875 * 2^9, that
    is e = x - 9, plus one when f > 0.875."""
    a = np.asarray(amax, np.float64)
    f, x = np.frexp(a)
    e = np.maximum(x - 9 + (f > 0.875), -126)
    return np.where(a > 0, np.ldexp(1.0, e), 1.0)


def nvis_of(lay, r):
    ns = np_i32(lay.n_slots)
    return np.minimum(ns[np_i32(lay.q_seq)], (np_i32(lay.q_pos) + 1) // r).clip(0)


# -------------------------------------------------------------------- compress
def run_compress(S, lay, lens):
    pre = torch.zeros((lay.cmp_blocks * 64, 576), dtype=torch.float32, device="cuda")
    S.compress(lay.ratio, lay.cu_seqlens, max(lens), lay.kv, lay.score, lay.gamma, lay.eps,
               lay.cos_sin, lay.cmp_pool, lay.cmp_table, prequant=pre)
    torch.cuda.synchronize()
    return pre


def compare_compress(lay, ref, pre, lens, r):
    """Rules: the pre-quant values within the fp32 rounding bound
    POOL_FP32_REL * M + 1e-5 |y| (M: pool_magnitude, the size of the terms a
    pooled value sums); codes, scales and bf16 rope dims equal except where
    the oracle's value lies within that same bound of a rounding midpoint
    (e4m3 or bf16) or of a scale boundary (counted), since a value decided
    in fp32 may then fall on the other side; the GPU's own codes / scales /
    rope are exactly the library casts of its pre-quant rows; no byte outside
    the produced slots is touched."""
    table = lay.cmp_table.cpu()
    pool = lay.cmp_pool.cpu()
    pre = pre.cpu().numpy()
    kv_all = lay.kv.cpu().float().numpy()
    sc_all = lay.score.cpu().numpy()
    gamma = lay.gamma.cpu().numpy().astype(np.float64)
    cu = lay.cu_seqlens.cpu().numpy()
    s0 = 0
    written = np.zeros(lay.cmp_blocks * 64, bool)
    excused = 0
    for b, L in enumerate(lens):
        n = -(-L // r)
        codes, scales, rope = P.cmp_pool_get(pool, table[b], 0, n)
        codes, scales, rope = codes.numpy(), scales.numpy(), bits16(rope)
        phys = (table[b].long()[torch.arange(n) // 64] * 64 + torch.arange(n) % 64).numpy()
        written[phys] = True
        g_pre = pre[phys]
        o_pre = ref["prequant"][s0:s0 + n]
        o_codes, o_scales, o_rope = ref["codes"][s0:s0 + n], ref["scales"][s0:s0 + n], ref["rope"][s0:s0 + n]
        t0 = int(cu[b])
        M = pool_magnitude(kv_all[t0:t0 + L], sc_all[t0:t0 + L], gamma, lay.eps, r)
        win_all = POOL_FP32_REL * M + 1e-5 * np.abs(o_pre.astype(np.float64))
        assert np.all(np.abs(g_pre.astype(np.float64) - o_pre) <= win_all)
        win = win_all[:, :512]
        # exactness of the GPU quantiser on its own pre-quant rows
        x = g_pre[:, :512].reshape(n, 8, 64).astype(np.float64)
        s_want = pow2_rule(np.max(np.abs(x), axis=2))
        assert np.array_equal(scales, s_want.astype(np.float32))
        want = torch.from_numpy((x / s_want[:, :, None]).astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes.reshape(n, 8, 64), want)
        assert np.array_equal(rope, bits16(torch.from_numpy(np.ascontiguousarray(g_pre[:, 512:]))))
        # against the oracle
        o_amax = np.max(np.abs(o_pre[:, :512].reshape(n, 8, 64)), axis=2)
        boundary = near_scale_boundary(o_amax, win=np.max(win.reshape(n, 8, 64), axis=2))
        assert np.all((scales == o_scales) | boundary)
        v = o_pre[:, :512].reshape(n, 8, 64) / o_scales[:, :, None]
        ok_elem = near_midpoint_within(v, win.reshape(n, 8, 64) / o_scales[:, :, None]) | \
            boundary[:, :, None]
        diff = codes.reshape(n, 8, 64) != o_codes.reshape(n, 8, 64)
        assert not np.any(diff & ~ok_elem), "fp8 code mismatch away from midpoints"
        excused += int(np.sum(diff))
        # rope dims: bf16 of the fp32 value; equal to the oracle's except where
        # its value lies within the fp32 bound of a bf16 rounding midpoint
        rdiff = rope != o_rope
        assert not np.any(rdiff & ~near_bf16_midpoint_within(o_pre[:, 512:], win_all[:, 512:])), \
            "rope mismatch away from bf16 midpoints"
        excused += int(np.sum(rdiff))
        s0 += n
    # untouched bytes: every row outside the produced slots is still zero
    rows, scl = pool.as_strided((lay.cmp_blocks, 64, 640), (43008, 640, 1)), \
        pool.as_strided((lay.cmp_blocks, 64, 32), (43008, 32, 1), 40960)
    rows = rows.reshape(-1, 640).numpy()
    scl = scl.reshape(-1, 32).numpy()
    assert not rows[~written].any() and not scl[~written].any()
    return excused


@pytest.mark.parametrize("r,lens", [(4, [37, 130, 1, 300, 4, 1029]),
                                    (128, [300, 129, 1000, 128, 5, 2049])])
def test_compress_matches_oracle(S, oracle, r, lens):
    n_slots = [-(-L // r) for L in lens]
    lay = I.build_layer(11, ratio=r, H=16, ctx=lens, queries=[(b, L - 1) for b, L in enumerate(lens)],
                        n_slots=n_slots, W=16, compress_inputs=True, gamma_random=True)
    ref = oracle_compress(oracle, lay)
    to_device(lay)
    pre = run_compress(S, lay, lens)
    excused = compare_compress(lay, ref, pre, lens, r)
    print(f"compress r={r}: {sum(n_slots)} slots, {excused} codes differ at midpoints")


@pytest.mark.parametrize("r,L", [(4, 65536), (128, 131072)], ids=["r4_65536", "r128_131072"])
def test_compress_full_length_matches_oracle(S, oracle, r, L):
    """One sequence at the decode workloads' full context: 65536 tokens at
    ratio 4 (16384 slots, 8-token overlapping windows) and 131072 tokens at
    ratio 128 (1024 slots), on permuted 64-slot blocks, by the same rules."""
    lay = I.build_layer(12, ratio=r, H=16, ctx=[L], queries=[(0, L - 1)], n_slots=[L // r],
                        W=16, compress_inputs=True, gamma_random=True)
    ref = oracle_compress(oracle, lay)
    to_device(lay)
    pre = run_compress(S, lay, [L])
    excused = compare_compress(lay, ref, pre, [L], r)
    print(f"compress r={r} L={L}: {L // r} slots, {excused} codes differ at midpoints")


def test_compress_truncates_to_max_seqlen_and_skips_absent_blocks(S, oracle):
    """max_seqlen = 300 of 500 tokens -> 75 slots; block 1 (slots 64..74) is absent:
    only block 0 may be written, and it holds the first 64 slots of the
    truncated sequence."""
    lay = I.build_layer(12, ratio=4, H=16, ctx=[500], queries=[(0, 499)], n_slots=[125], W=16,
                        compress_inputs=True)
    ref = oracle.compress_seq(4, bits16(lay.kv[:300]), np_f32(lay.score[:300]), np_f32(lay.gamma),
                              lay.eps, np_f32(lay.cos_sin))
    table = lay.cmp_table.clone()
    table[0, 1] = -1
    lay.cmp_table = table
    to_device(lay)
    S.compress(4, lay.cu_seqlens, 300, lay.kv, lay.score, lay.gamma, lay.eps, lay.cos_sin,
               lay.cmp_pool, lay.cmp_table)
    torch.cuda.synchronize()
    pool = lay.cmp_pool.cpu()
    t = lay.cmp_table.cpu()
    codes, scales, _ = P.cmp_pool_get(pool, t[0], 0, 64)
    for blk in range(lay.cmp_blocks):
        if blk != int(t[0, 0]):
            assert not pool[blk].any()
    assert np.all(scales.numpy() == ref["scales"][:64])
    diff = codes.numpy() != ref["codes"][:64]
    assert np.mean(diff) < 1e-3


# ------------------------------------------------------------------ indexer
@pytest.mark.parametrize("h_idx", [16, 64])
def test_index_scores_and_topk_match_oracle(S, oracle, h_idx):
    lay = I.build_layer(13, ratio=4, H=16, ctx=[1200, 4000, 333],
                        queries=[(0, 1199), (0, 600), (1, 3999), (1, 16), (2, 332), (2, 2), (1, 2047)],
                        n_slots=[300, 1000, 84], W=16, k=64, H_I=h_idx)
    idx_ref, len_ref, sc_ref = oracle_index_topk(oracle, lay)
    to_device(lay)
    sc, idx, ln = gpu_index_topk(S, lay)
    torch.cuda.synchronize()
    sc, idx, ln = sc.cpu().numpy(), idx.cpu().numpy(), ln.cpu().numpy()
    nv = nvis_of(lay, 4)
    for t in range(lay.n_q):
        n = nv[t]
        o = sc_ref[t, :n].astype(np.float64)
        g = sc[t, :n].astype(np.float64)
        assert np.all(np.abs(g - o) <= 1e-5 * np.abs(o) + 1e-7 * max(1e-30, np.max(np.abs(o), initial=0)))
        assert np.all(np.isnan(sc[t, n:]))               # nothing past n_vis is written
    assert np.array_equal(ln, len_ref)
    near = check_topk_sets(idx, ln, sc_ref, nv, lay.k)
    # the GPU's selection is exactly the top-k of its own scores, in slot order
    assert np.array_equal(idx, exact_topk_of(sc, nv, lay.k))
    print(f"h_idx={h_idx}: near-tie slots excluded: {near}")


def test_index_topk_at_the_maxima(S, oracle):
    """64 index heads and k = 4096 (the ABI's maxima), with lists longer and
    shorter than k."""
    lay = I.build_layer(21, ratio=4, H=16, ctx=[40000, 12000],
                        queries=[(0, 39999), (1, 11999), (0, 16383)], n_slots=[10000, 3000],
                        W=16, k=4096, H_I=64)
    idx_ref, len_ref, sc_ref = oracle_index_topk(oracle, lay)
    to_device(lay)
    sc, idx, ln = gpu_index_topk(S, lay)
    torch.cuda.synchronize()
    sc, idx, ln = sc.cpu().numpy(), idx.cpu().numpy(), ln.cpu().numpy()
    nv = nvis_of(lay, 4)
    assert np.array_equal(ln, len_ref) and list(ln) == [4096, 3000, 4096]
    check_topk_sets(idx, ln, sc_ref, nv, lay.k)
    assert np.array_equal(idx, exact_topk_of(sc, nv, lay.k))


@pytest.mark.parametrize("key_fp4", [False, True], ids=["fp8_keys", "mxfp4_keys"])
def test_index_scores_multi_query_tiles(S, oracle, key_fp4):
    """A grid large enough for the prefill form of the index kernel (several
    queries per workgroup sharing key loads): 301 queries, so the last
    workgroup has one; neighbouring queries of one sequence (shared keys) and
    of different sequences (a pass each), causal counts that differ between
    the workgroup's queries, and queries that see no slot."""
    rng = np.random.default_rng(5)
    ctx = [10000, 6000, 2500]
    queries = []
    for i in range(301):
        if i % 4 < 2:                                   # a pair of adjacent tokens of one sequence
            b = (i // 4) % 3
            p0 = int(rng.integers(0, ctx[b] - 1)) if i % 4 == 0 else queries[-1][1] + 1
            queries.append((b, min(p0, ctx[b] - 1)))
        else:                                           # a pair across sequences
            b = i % 3
            queries.append((b, int(rng.integers(0, ctx[b]))))
    queries[7] = (queries[6][0], 1)                     # sees no slot, beside a query that does
    lay = I.build_layer(23, ratio=4, H=16, ctx=ctx, queries=queries, n_slots=[2500, 1500, 625],
                        W=16, k=128, H_I=16, key_fp4=key_fp4)
    idx_ref, len_ref, sc_ref = oracle_index_topk(oracle, lay)
    to_device(lay)
    assert lay.n_q * ((lay.max_slots + 2047) // 2048) > 512    # the multi-query form
    sc, idx, ln = gpu_index_topk(S, lay)
    torch.cuda.synchronize()
    sc, idx, ln = sc.cpu().numpy(), idx.cpu().numpy(), ln.cpu().numpy()
    nv = nvis_of(lay, 4)
    for t in range(lay.n_q):
        n = nv[t]
        o = sc_ref[t, :n].astype(np.float64)
        g = sc[t, :n].astype(np.float64)
        assert np.all(np.abs(g - o) <= 1e-5 * np.abs(o) + 1e-7 * max(1e-30, np.max(np.abs(o), initial=0))), t
        assert np.all(np.isnan(sc[t, n:])), t              # nothing past n_vis is written
    assert np.array_equal(ln, len_ref)
    check_topk_sets(idx, ln, sc_ref, nv, lay.k)
    assert np.array_equal(idx, exact_topk_of(sc, nv, lay.k))


@pytest.mark.parametrize("key_fp4", [False, True], ids=["fp8_keys", "mxfp4_keys"])
def test_index_scores_multi_query_spans(S, oracle, key_fp4):
    """The prefill form of the index kernel over rows longer than one span of
    a workgroup's blocks: 9000 and 5200 slots, so workgroups take a second
    span (and stop early where their queries see fewer slots), with pairs of
    one sequence (shared keys) and pairs across sequences (a pass each, in
    every span)."""
    rng = np.random.default_rng(8)
    ctx = [36000, 20800]
    queries = []
    for i in range(520):
        if i % 4 < 2:                                   # a pair of adjacent tokens of one sequence
            b = (i // 4) % 2
            p0 = int(rng.integers(ctx[b] // 2, ctx[b] - 1)) if i % 4 == 0 else queries[-1][1] + 1
            queries.append((b, min(p0, ctx[b] - 1)))
        else:                                           # a pair across sequences
            b = i % 2
            queries.append((b, int(rng.integers(0, ctx[b]))))
    lay = I.build_layer(24, ratio=4, H=16, ctx=ctx, queries=queries, n_slots=[9000, 5200],
                        W=16, k=128, H_I=16, key_fp4=key_fp4)
    idx_ref, len_ref, sc_ref = oracle_index_topk(oracle, lay)
    to_device(lay)
    assert lay.n_q * ((lay.max_slots + 2047) // 2048) > 512    # the multi-query form
    sc, idx, ln = gpu_index_topk(S, lay)
    torch.cuda.synchronize()
    sc, idx, ln = sc.cpu().numpy(), idx.cpu().numpy(), ln.cpu().numpy()
    nv = nvis_of(lay, 4)
    assert nv.max() > 8192                              # some workgroups reach a third 4096-slot run
    for t in range(lay.n_q):
        n = nv[t]
        o = sc_ref[t, :n].astype(np.float64)
        g = sc[t, :n].astype(np.float64)
        assert np.all(np.abs(g - o) <= 1e-5 * np.abs(o) + 1e-7 * max(1e-30, np.max(np.abs(o), initial=0))), t
        assert np.all(np.isnan(sc[t, n:])), t              # nothing past n_vis is written
    assert np.array_equal(ln, len_ref)
    check_topk_sets(idx, ln, sc_ref, nv, lay.k)
    assert np.array_equal(idx, exact_topk_of(sc, nv, lay.k))


@pytest.mark.parametrize("H", [16, 48])
def test_topk_select_warm_equals_select(S, oracle, H):
    """The select with the decode's L2 warm-up (extra read-only workgroups) gives
    the plain select's lists bit for bit, on lists long enough for the main
    select kernel, with windows that reach before position 0."""
    lay = I.build_layer(19, ratio=4, H=H, ctx=[12000, 9000],
                        queries=[(0, 11999), (0, 5), (1, 8999), (1, 100), (0, 130)],
                        n_slots=[3000, 2250], W=128, k=64, H_I=16)
    to_device(lay)
    sc, idx, ln = gpu_index_topk(S, lay)
    idx_w = torch.full_like(idx, -7)
    ln_w = torch.full_like(ln, -7)
    S.topk_select_warm(lay.k, sc, lay.max_slots, lay.q_seq, lay.q_pos, 4, lay.n_slots, idx_w, ln_w,
                       lay.q, lay.W, lay.swa_pool, lay.swa_table)
    torch.cuda.synchronize()
    assert lay.max_slots > 2048
    assert torch.equal(idx_w, idx) and torch.equal(ln_w, ln)


def test_topk_ties_and_short_lists(S, oracle):
    lay = I.build_layer(14, ratio=4, H=16, ctx=[2000, 40],
                        queries=[(0, 1999), (0, 2), (1, 39), (0, 100)], n_slots=[500, 10], W=16,
                        k=32, H_I=16)
    lay.qi = torch.zeros_like(lay.qi)       # every score is exactly 0: lowest slots win
    idx_ref, len_ref, _ = oracle_index_topk(oracle, lay)
    to_device(lay)
    sc, idx, ln = gpu_index_topk(S, lay)
    idx, ln = idx.cpu().numpy(), ln.cpu().numpy()
    assert np.array_equal(ln, [32, 0, 10, 25])
    assert np.array_equal(idx, idx_ref)
    assert np.array_equal(idx[0], np.arange(32)) and np.all(idx[1] == -1)
    assert np.array_equal(idx[2, :10], np.arange(10)) and np.all(idx[2, 10:] == -1)


def test_topk_beyond_lds_capacity(S, oracle):
    """More visible slots than the top-k kernel caches in LDS (global-memory path)."""
    lay = I.build_layer(15, ratio=4, H=16, ctx=[160000], queries=[(0, 159999), (0, 150003)],
                        n_slots=[40000], W=16, k=700, H_I=16)
    idx_ref, len_ref, sc_ref = oracle_index_topk(oracle, lay)
    to_device(lay)
    sc, idx, ln = gpu_index_topk(S, lay)
    sc, idx, ln = sc.cpu().numpy(), idx.cpu().numpy(), ln.cpu().numpy()
    nv = nvis_of(lay, 4)
    check_topk_sets(idx, ln, sc_ref, nv, lay.k)
    assert np.array_equal(idx, exact_topk_of(sc, nv, lay.k))


def _crafted_rows():
    """Score rows built to drive each threshold path of the select: a crowded
    bin of exact ties, a crowded bin of distinct keys (several radix passes),
    a range so narrow that a bin is one key, -inf / -0 / +0 mixes, wide
    random ranges, and k at both extremes."""
    rng = np.random.default_rng(7)
    f32 = np.float32
    rows = []
    n = 16384
    v = rng.uniform(0.0, 0.74, n).astype(f32)
    ties = rng.choice(n, 2300, replace=False)
    v[ties[:300]] = rng.uniform(0.76, 1.0, 300).astype(f32)
    v[ties[300:]] = f32(0.75)
    rows.append(("crowded_ties", v, 512))
    n = 8192
    v = np.full(n, 1e-20, f32)
    pos = rng.permutation(n)
    v[pos[:500]] = f32(1e20)
    v[pos[500:3500]] = (np.float32(1.0).view(np.int32) + rng.permutation(3000)).astype(np.int32).view(f32)
    rows.append(("crowded_distinct", v, 1000))
    n = 4096
    v = (np.float32(1.0).view(np.int32) + rng.integers(0, 600, n)).astype(np.int32).view(f32)
    rows.append(("narrow_ties", v, 100))
    n = 5000
    v = -rng.uniform(0.1, 10.0, n).astype(f32)
    pos = rng.permutation(n)
    v[pos[:1000]] = -np.inf
    v[pos[1000:1500]] = f32(-0.0)
    v[pos[1500:2000]] = f32(0.0)
    v[pos[2000:2300]] = rng.uniform(0.1, 5.0, 300).astype(f32)
    rows.append(("inf_and_signed_zeros", v, 700))
    n = 40000
    v = (rng.lognormal(0.0, 4.0, n) * rng.choice([-1.0, 1.0], n)).astype(f32)
    rows.append(("wide_random_40k", v, 4096))
    n = 20000
    v = rng.integers(0, 50, n).astype(f32)
    rows.append(("k1_with_ties", v, 1))
    n = 1000
    v = rng.normal(size=n).astype(f32)
    rows.append(("k_n_minus_1", v, 999))
    n = 777
    v = rng.normal(size=n).astype(f32)
    rows.append(("short_row", v, 300))
    # full rows, where every wave of the select bounds the threshold by
    # itself: the top keys concentrated in the first waves' slots, and heavy
    # ties everywhere
    n = 16384
    v = rng.uniform(0.0, 1.0, n).astype(f32)
    v[rng.permutation(2000)[:600]] = (2.0 + rng.uniform(0.0, 1.0, 600)).astype(f32)
    rows.append(("wave_bound_concentrated", v, 512))
    n = 16384
    v = rng.integers(0, 41, n).astype(f32)
    rows.append(("wave_bound_ties", v, 512))
    # past 65536 slots (the long-row kernel): a 1M-token context at ratio 4 is
    # 262144 slots; heavy exact ties at the threshold, -inf and signed zeros
    n = 262144
    v = rng.normal(size=n).astype(f32)
    rows.append(("long_262144_k512", v, 512))
    n = 262144
    v = rng.uniform(0.0, 0.5, n).astype(f32)
    pos = rng.permutation(n)
    v[pos[:1500]] = rng.uniform(0.6, 1.0, 1500).astype(f32)
    v[pos[1500:9000]] = f32(0.55)                       # the threshold: 7500 equal keys
    v[pos[9000:30000]] = -np.inf
    v[pos[30000:30100]] = f32(-0.0)
    rows.append(("long_262144_ties_k2048", v, 2048))
    n = 70000
    v = (np.float32(1.0).view(np.int32) + rng.integers(0, 3000, n)).astype(np.int32).view(f32)
    rows.append(("long_70000_narrow_k4096", v, 4096))
    n = 65537
    v = -np.abs(rng.normal(size=n)).astype(f32)
    v[rng.permutation(n)[:40000]] = f32(0.0)            # ties of zeros straddle the threshold
    rows.append(("long_65537_zero_ties_k4096", v, 4096))
    return rows


@pytest.mark.parametrize("name,row,k", _crafted_rows(), ids=[r[0] for r in _crafted_rows()])
def test_topk_crafted_rows_match_oracle(S, oracle, name, row, k):
    n = row.shape[0]
    ref_idx, ref_len = oracle.topk(row, k)
    sc = torch.from_numpy(row.reshape(1, n)).cuda()
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    ln = torch.empty(1, dtype=torch.int32, device="cuda")
    S.topk_select(k, sc, n, one, torch.full((1,), 4 * n - 1, dtype=torch.int32, device="cuda"),
                  4, torch.full((1,), n, dtype=torch.int32, device="cuda"), idx, ln)
    torch.cuda.synchronize()
    g = idx.cpu().numpy()[0]
    assert int(ln.item()) == ref_len == min(k, n)
    assert np.array_equal(g[:ref_len], np.sort(ref_idx[:ref_len])), name
    assert np.all(g[ref_len:] == -1)


# --------------------------------------------------------------- attention
def _noisy_idx(lay, seed=0):
    """Given lists with -1, out-of-range entries and a duplicate mixed in."""
    idx = lay.given_idx.clone()
    g = torch.Generator().manual_seed(seed)
    for t in range(idx.shape[0]):
        j = torch.randint(0, idx.shape[1], (3,), generator=g)
        idx[t, j[0]] = -1
        idx[t, j[1]] = 10 ** 6
        idx[t, j[2]] = idx[t, (int(j[2]) + 1) % idx.shape[1]]
    return idx


ATTN_CASES = {
    "swaonly_h16": dict(ratio=1, H=16, ctx=[500, 90, 1000], queries=[(0, 499), (1, 89), (2, 999)],
                        n_slots=[0, 0, 0], W=128),
    "swaonly_h64_w200": dict(ratio=1, H=64, ctx=[500, 300], queries=[(0, 499), (1, 150)],
                             n_slots=[0, 0], W=200),
    "c128a_h64": dict(ratio=128, H=64, ctx=[40000, 9000], queries=[(0, 39999), (1, 8999)],
                      n_slots=[313, 71], W=128, k=100, given_topk=True),
    "c4a_given_h16": dict(ratio=4, H=16, ctx=[4000, 700, 1500],
                          queries=[(0, 3999), (1, 699), (2, 1499)], n_slots=[1000, 175, 375],
                          W=128, k=256, given_topk=True),
    "c4a_given_h48": dict(ratio=4, H=48, ctx=[4000], queries=[(0, 3999)], n_slots=[1000], W=64,
                          k=77, given_topk=True),
    # head counts whose 16-head groups split into uneven blocks of four:
    # 80 heads run as five blocks of 16, 96 as two blocks of 48
    "c4a_given_h80": dict(ratio=4, H=80, ctx=[3000, 900], queries=[(0, 2999), (1, 899)],
                          n_slots=[750, 225], W=96, k=130, given_topk=True),
    "c4a_given_h96": dict(ratio=4, H=96, ctx=[2500], queries=[(0, 2499)], n_slots=[625], W=128,
                          k=200, given_topk=True),
    # the ABI's maxima: 128 heads, a 1024-row window, a 4096-entry list
    "c4a_max_h128_w1024_k4096": dict(ratio=4, H=128, ctx=[20000, 1500],
                                     queries=[(0, 19999), (1, 1499)], n_slots=[5000, 375],
                                     W=1024, k=4096, given_topk=True),
}


@pytest.mark.parametrize("decode", [True, False], ids=["decode", "prefill"])
@pytest.mark.parametrize("case", list(ATTN_CASES))
def test_attention_matches_oracle(S, oracle, case, decode):
    lay = I.build_layer(16, **ATTN_CASES[case])
    idx = _noisy_idx(lay) if lay.given_idx is not None else None
    out_ref, lse_ref = oracle_attention(oracle, lay, None if idx is None else idx.numpy())
    to_device(lay)
    out, lse = gpu_attention(S, lay, None if idx is None else idx.cuda(), decode=decode)
    torch.cuda.synchronize()
    errs = check_attention(out, lse, out_ref, lse_ref)
    print(f"{case} decode={decode}: max abs {errs[0]:.3g} rel L2 {errs[1]:.3g} lse {errs[2]:.3g}")


def test_prefill_many_queries_matches_oracle(S, oracle):
    lay = I.build_layer(17, ratio=4, H=64, ctx=[3000], queries=[(0, p) for p in range(2800, 3000, 7)],
                        n_slots=[750], W=128, k=200, given_topk=True)
    out_ref, lse_ref = oracle_attention(oracle, lay, lay.given_idx.numpy())
    to_device(lay)
    out, lse = gpu_attention(S, lay, lay.given_idx, decode=False)
    check_attention(out, lse, out_ref, lse_ref)
    out2, lse2 = gpu_attention(S, lay, lay.given_idx, decode=True)
    check_attention(out2, lse2, out_ref, lse_ref)


def test_empty_lists_give_zero_and_minus_inf(S, oracle):
    lay = I.build_layer(18, ratio=128, H=16, ctx=[1000], queries=[(0, 999)], n_slots=[7], W=0,
                        k=4, given_topk=True)
    idx = torch.full((1, 4), -1, dtype=torch.int32)
    to_device(lay)
    out, lse = gpu_attention(S, lay, idx.cuda())
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_paging_is_bit_identical(S):
    """Contiguous and randomly permuted block tables give identical bits."""
    res = []
    for permute in (False, True):
        lay = I.build_layer(19, ratio=4, H=64, ctx=[9000, 5000], queries=[(0, 8999), (1, 4999)],
                            n_slots=[2250, 1250], W=128, k=300, H_I=64, permute=permute)
        to_device(lay)
        sc, idx, ln = gpu_index_topk(S, lay)
        out, lse = gpu_attention(S, lay, idx)
        res.append([x.cpu() for x in (sc, idx, ln, out, lse)])
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a, b.view(
            torch.uint8) if b.dtype == torch.bfloat16 else b) or torch.equal(a.nan_to_num(), b.nan_to_num())


def test_repeated_runs_are_bitwise_deterministic(S):
    lay = I.build_layer(20, ratio=4, H=64, ctx=[20000] * 3, queries=[(b, 19999) for b in range(3)],
                        n_slots=[5000] * 3, W=128, k=512, H_I=64)
    to_device(lay)
    runs = []
    for _ in range(2):
        sc, idx, ln = gpu_index_topk(S, lay)
        out, lse = gpu_attention(S, lay, idx)
        runs.append((sc.cpu(), idx.cpu(), out.cpu().view(torch.int16), lse.cpu()))
    for a, b in zip(*runs):
        assert torch.equal(a.nan_to_num(), b.nan_to_num()) if a.is_floating_point() else torch.equal(a, b)


# ------------------------------------------------------------- whole chain
def test_c4a_single_layer_chain(S, oracle):
    """C4A single-layer decode, batch 1 (H=16, context 4096 -> 1024 slots, top-k
    256, SWA 128): compress -> index top-k -> sparse decode, each stage
    checked against the oracle's own chain."""
    lay = I.c4a_single_layer_4k()
    ref = oracle_compress(oracle, lay)
    idx_ref, len_ref, sc_ref = oracle_index_topk(oracle, lay)
    out_ref, lse_ref = oracle_attention(oracle, lay, idx_ref,
                                        cmp=dict(codes=ref["codes"], scales=ref["scales"],
                                                 rope=ref["rope"]))
    to_device(lay)
    pre = run_compress(S, lay, [4096])
    compare_compress(lay, ref, pre, [4096], 4)
    sc, idx, ln = gpu_index_topk(S, lay)
    nv = nvis_of(lay, 4)
    check_topk_sets(idx.cpu().numpy(), ln.cpu().numpy(), sc_ref, nv, lay.k)
    out, lse = gpu_attention(S, lay, idx)
    check_attention(out, lse, out_ref, lse_ref)
