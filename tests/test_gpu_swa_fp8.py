"""GPU parity of the fp8 sliding-window pool ("From MLA to CSA + HCA" 5.5 and
6.2): the SWA KV insert (RoPE at each token's position, the fp8 row format,
paged write) against the oracle's insert, and sparse MLA decode / prefill over
an fp8 SWA pool against the oracle attending to the rows that pool stands
for.  The insert's nope dims pass through no arithmetic before quantisation,
so their codes and scales must match bit for bit; the rope dims may differ by
the fp32 rounding of the rotation (one bf16 step at most)."""
import numpy as np
import pytest
import torch

from helpers import (bits16, check_attention, check_attention_scaled, check_topk_sets,
                     gpu_attention, gpu_index_topk, np_f32, np_i32, np_u8, oracle_attention,
                     oracle_index_topk, to_device, value_absmax)
from sparse_long_context_compressor_amd import inputs as I
from sparse_long_context_compressor_amd import pools as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    from sparse_long_context_compressor_amd import slc
    slc.lib()
    return slc


def _bf16_ulps(a_bits, b_bits):
    """|a - b| in bf16 steps for same-sign finite values given as bits."""
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    sa, sb = a >> 15, b >> 15
    ma, mb = a & 0x7FFF, b & 0x7FFF
    return np.where(sa == sb, np.abs(ma - mb), ma + mb)


def _kv(n, seed, spread=2.0):
    """Latent rows whose 64-dim blocks have magnitudes e^(spread * N(0,1))."""
    g = torch.Generator().manual_seed(seed)
    scale = torch.exp(torch.randn((n, 9), generator=g) * spread).repeat_interleave(64, dim=1)
    return (torch.randn((n, 576), generator=g) * scale).to(torch.bfloat16)


def _insert_case(seed=5):
    ctx = [300, 130, 70]
    toks = ([(0, p) for p in (0, 1, 63, 64, 65, 127, 128, 150, 191, 192, 255, 299)] +
            [(1, p) for p in range(0, 130, 7)] + [(2, p) for p in range(58, 70)])
    blocks = [list(range(-(-L // 64))) for L in ctx]
    table, nb = I.block_table(blocks, 5, seed, "swa8_table", "cpu", True)
    table[0, 2] = -1                         # positions 128..191 of sequence 0 have no block
    seq = torch.tensor([s for s, _ in toks], dtype=torch.int32)
    pos = torch.tensor([p for _, p in toks], dtype=torch.int32)
    kv = _kv(len(toks), seed)
    # one token's first 64-dim block is denormal-sized: its scale stops at
    # 2^-126, the smallest normal fp32 power of two
    kv[2, :64] = (kv[2, :64].float() * 2.0 ** -132).to(torch.bfloat16)
    return toks, table, nb, seq, pos, kv


def test_swa_insert_matches_oracle(S, oracle):
    toks, table, nb, seq, pos, kv = _insert_case()
    cs = I.rope_table(320)
    codes, scales, rope, pre = oracle.swa_insert(bits16(kv), pos.numpy(), cs.numpy())
    dev = "cuda"
    pool = P.cmp_pool_empty(nb, dev)
    pq = torch.full((len(toks), 576), float("nan"), device=dev)
    S.swa_insert(kv.to(dev), seq.to(dev), pos.to(dev), cs.to(dev), pool, table.to(dev), pq)
    torch.cuda.synchronize()
    pool, pq = pool.cpu(), pq.cpu().numpy()
    # the row before quantisation: nope dims exact, rope dims to the fp32
    # rounding of a rotation (a few steps of the pair's norm, which the
    # rotation keeps)
    assert np.array_equal(pq[:, :512], pre[:, :512])
    pair = np.repeat(np.hypot(pre[:, 512::2].astype(np.float64), pre[:, 513::2]), 2, axis=1)
    rd = np.abs(pq[:, 512:].astype(np.float64) - pre[:, 512:])
    assert np.all(rd <= 4 * np.spacing(pair.astype(np.float32)) + 1e-38)
    big = np.abs(pre[:, 512:]) >= pair / 64      # no cancellation in the rotation
    written = np.zeros((nb, 64), bool)
    for t, (s, p) in enumerate(toks):
        pb = int(table[s, p // 64])
        if pb < 0:
            continue
        written[pb, p % 64] = True
        c, sc, rp = P.cmp_pool_get(pool, table[s], p, 1)
        assert np.array_equal(c.numpy()[0], codes[t]), f"token {t}: codes"
        assert np.array_equal(sc.numpy()[0], scales[t]), f"token {t}: scales"
        assert np.all(_bf16_ulps(bits16(rp)[0], rope[t])[big[t]] <= 1), f"token {t}: rope"
        # the stored rope is the bf16 rounding of the kernel's own fp32 row
        assert np.array_equal(bits16(rp)[0], bits16(torch.from_numpy(pq[t, 512:])))
    # nothing else in the pool was touched (absent blocks included)
    rows, scl = P._cmp_views(pool)
    assert not rows[torch.from_numpy(~written)].any()
    assert not scl[torch.from_numpy(~written)].any()
    assert written.sum() == sum(1 for s, p in toks if int(table[s, p // 64]) >= 0) < len(toks)


SWA8_CASES = {
    "c4a_H16_ragged": dict(ratio=4, H=16, ctx=[700, 90], queries=[(0, 699), (1, 89), (0, 40)],
                           n_slots=[175, 22], W=128, k=64),
    "c128a_H64": dict(ratio=128, H=64, ctx=[20000], queries=[(0, 19999), (0, 12000)],
                      n_slots=[156], W=128, k=96, given_topk=True),
    "swaonly_H32_W300": dict(ratio=1, H=32, ctx=[1000, 250], queries=[(0, 999), (1, 249), (1, 5)],
                             n_slots=[0, 0], W=300),
}


def _list_of(lay):
    if lay.ratio == 1:
        return None
    if lay.given_idx is not None:
        return lay.given_idx
    g = torch.Generator().manual_seed(7)
    idx = torch.full((lay.n_q, lay.k), -1, dtype=torch.int32)
    for t in range(lay.n_q):
        ns = int(lay.n_slots[int(lay.q_seq[t])])
        vis = min(ns, (int(lay.q_pos[t]) + 1) // lay.ratio)
        perm = torch.randperm(max(vis, 1), generator=g)[:min(lay.k, vis)]
        idx[t, :perm.numel()] = perm.to(torch.int32)
    return idx


@pytest.mark.parametrize("decode", [True, False], ids=["decode", "prefill"])
@pytest.mark.parametrize("case", list(SWA8_CASES))
def test_attention_over_fp8_swa_matches_oracle(S, oracle, case, decode):
    lay = I.build_layer(60, swa_fp8=True, **SWA8_CASES[case])
    idx = _list_of(lay)
    out_ref, lse_ref = oracle_attention(oracle, lay, None if idx is None else idx.numpy())
    to_device(lay)
    out, lse = gpu_attention(S, lay, None if idx is None else idx.to("cuda"), decode=decode)
    torch.cuda.synchronize()
    check_attention(out, lse, out_ref, lse_ref)


@pytest.mark.parametrize("decode", [True, False], ids=["decode", "prefill"])
@pytest.mark.parametrize("case", list(SWA8_CASES))
def test_attention_over_wide_scale_fp8_swa(S, oracle, case, decode):
    """fp8 SWA rows whose 64-dim blocks take scales 2^-8 .. 2^-5 (so that a
    per-block scale addressing slip changes the result), judged by the bar
    that scales with the rows' values (check_attention_scaled): |g - o| <=
    2e-2 + 2^-8 max|V_d| + one bf16 step at |o|, relative L2 <= 1e-2, lse
    within 2e-2."""
    lay = I.build_layer(64, swa_fp8=True, swa_scale_exp=(-8, -5), **SWA8_CASES[case])
    sc = np_f32(lay.swa_scales)
    assert len(np.unique(sc)) == 4 and np.any(sc[:, :, None] != sc[:, None, :])
    idx = _list_of(lay)
    out_ref, lse_ref = oracle_attention(oracle, lay, None if idx is None else idx.numpy())
    vmax = value_absmax(oracle, lay, None if idx is None else idx.numpy())
    to_device(lay)
    out, lse = gpu_attention(S, lay, None if idx is None else idx.to("cuda"), decode=decode)
    torch.cuda.synchronize()
    e = check_attention_scaled(out, lse, out_ref, lse_ref, vmax)
    print(f"{case} wide scales: max abs {e[0]:.3g} (max |o| {e[3]:.3g}, max |V| {e[4]:.3g}), "
          f"rel L2 {e[1]:.3g}")


@pytest.mark.parametrize("spread", [0.25, 2.0], ids=["unit_scale", "wide_scale"])
def test_insert_then_decode_chain(S, oracle, spread):
    """New tokens' rows go through the insert into an fp8 pool and the decode
    attends to them: the oracle's insert feeds the oracle's attention, the
    kernel's insert feeds the kernel's decode."""
    lay = I.build_layer(61, ratio=4, H=64, ctx=[5000, 3000], queries=[(0, 4999), (1, 2999)],
                        n_slots=[1250, 750], W=128, k=128, swa_fp8=True)
    idx = _list_of(lay)
    cs = I.rope_table(5000)
    counts = np_i32(lay.swa_count)
    seq = np.repeat(np.arange(lay.n_seq, dtype=np.int32), counts)
    pos = np.concatenate([np.arange(b, b + c, dtype=np.int32)
                          for b, c in zip(np_i32(lay.swa_base), counts)])
    # unit-scale rows, as a normed latent is; and rows whose 64-dim blocks
    # span magnitudes e^(2 N(0,1)), judged by the bar that scales with |o|
    kv = _kv(len(pos), 62, spread=spread)
    codes, scales, rope, _ = oracle.swa_insert(bits16(kv), pos, cs.numpy())
    lay.swa_codes = torch.from_numpy(codes)
    lay.swa_scales = torch.from_numpy(scales)
    lay.swa_rope = torch.from_numpy(rope.view(np.int16)).view(torch.bfloat16)
    out_ref, lse_ref = oracle_attention(oracle, lay, idx.numpy())
    vmax = value_absmax(oracle, lay, idx.numpy())
    to_device(lay)
    lay.swa_pool.zero_()
    S.swa_insert(kv.cuda(), torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), cs.cuda(),
                 lay.swa_pool, lay.swa_table)
    out, lse = gpu_attention(S, lay, idx.cuda())
    torch.cuda.synchronize()
    if spread < 1.0:
        check_attention(out, lse, out_ref, lse_ref)
    else:
        e = check_attention_scaled(out, lse, out_ref, lse_ref, vmax)
        print(f"wide-scale chain: max abs {e[0]:.3g} (max |o| {e[3]:.3g}, max |V| {e[4]:.3g}), "
              f"rel L2 {e[1]:.3g}")


def test_warm_select_over_fp8_swa_equals_select(S, oracle):
    """The select's L2 warm-up reads the fp8 pool's layout; lists unchanged."""
    lay = I.build_layer(63, ratio=4, H=48, ctx=[12000, 9000], queries=[(0, 11999), (1, 8999)],
                        n_slots=[3000, 2250], W=128, k=256, H_I=16, swa_fp8=True)
    _, _, sc_ref = oracle_index_topk(oracle, lay)
    to_device(lay)
    sc, idx, ln = gpu_index_topk(S, lay)
    idx_w = torch.full_like(idx, -7)
    ln_w = torch.full_like(ln, -7)
    S.topk_select_warm(lay.k, sc, lay.max_slots, lay.q_seq, lay.q_pos, 4 | S.SWA_FP8, lay.n_slots,
                       idx_w, ln_w, lay.q, lay.W, lay.swa_pool, lay.swa_table)
    torch.cuda.synchronize()
    assert torch.equal(idx_w, idx) and torch.equal(ln_w, ln)
    nv = np.minimum((np_i32(lay.q_pos) + 1) // 4, np_i32(lay.n_slots)[np_i32(lay.q_seq)])
    check_topk_sets(idx.cpu().numpy(), ln.cpu().numpy(), sc_ref, nv, lay.k)
