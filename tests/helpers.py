"""Shared test helpers: run the CPU oracle and the HIP library on the same
seeded workload, and the acceptance rules both are judged by."""
from __future__ import annotations

import numpy as np
import torch

from sparse_long_context_compressor_amd import pools as P


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns (float tensors of other dtypes are rounded to bf16 first)."""
    t = t.detach().to("cpu")
    if t.dtype not in (torch.bfloat16, torch.int16):
        t = t.to(torch.bfloat16)
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def np_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy().astype(np.uint8, copy=False)


def np_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy().astype(np.float32, copy=False)


def np_i32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().numpy().astype(np.int32, copy=False)


def fp8_values(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


_E4M3 = None


def e4m3_midpoints():
    global _E4M3
    if _E4M3 is None:
        v = np.unique(np.abs(fp8_values(np.arange(0, 0x7F, dtype=np.uint8))))
        _E4M3 = (v[:-1] + v[1:]) / 2
    return _E4M3


def near_midpoint(x: np.ndarray, rel=1e-5) -> np.ndarray:
    """True where |x| lies within rel (relative) of an e4m3 rounding midpoint."""
    mids = e4m3_midpoints()
    a = np.abs(x.astype(np.float64))
    j = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    d = np.minimum(np.abs(a - mids[j - 1]), np.abs(a - mids[j]))
    return d <= rel * np.maximum(a, 1e-30)


def near_scale_boundary(amax: np.ndarray, rel=1e-5, win=None) -> np.ndarray:
    """True where amax lies within rel (relative) plus win (absolute, same
    shape, optional) of some 448 * 2^e."""
    a = np.maximum(amax.astype(np.float64), 1e-300)
    e = np.round(np.log2(a / 448.0))
    b = 448.0 * np.exp2(e)
    return np.abs(a - b) <= rel * a + (0.0 if win is None else win)


def near_midpoint_within(v: np.ndarray, win: np.ndarray) -> np.ndarray:
    """True where |v| lies within win (absolute, same shape) of an e4m3
    rounding midpoint."""
    mids = e4m3_midpoints()
    a = np.abs(v.astype(np.float64))
    j = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    d = np.minimum(np.abs(a - mids[j - 1]), np.abs(a - mids[j]))
    return d <= win


# Relative size of the fp32 rounding in a compressed row before quantisation,
# against the size of the terms it sums (see pool_magnitude): the window
# weights' exponent arguments and exp (a few ulp of |s - m| <= ~10), the
# window sum and the RMSNorm divisor over 576 dims come to a few 1e-6 at most;
# 2^-16 (1.5e-5) leaves a margin over that.
POOL_FP32_REL = 2.0 ** -16


def pool_magnitude(kv: np.ndarray, score: np.ndarray, gamma: np.ndarray, eps: float, r: int,
                   chunk: int = 128) -> np.ndarray:
    """Per slot of one sequence (kv [L,576] values, score [L,576]) and dim:
    M = gamma * (sum_t w_t |kv_t|) / (sum_t w_t) / rms, with w_t the window's
    per-channel softmax weights and rms the slot's RMSNorm divisor, so that
    |y| <= M (for the rope dims, the sum over the rotated pair).  The fp32 rounding of a pooled value is bounded relative to M,
    not to |y|: the weights' rounding scales every term, and the terms can
    cancel.  Windows as the compressor's (r = 4: [4j-4, 4j+3]; r = 128:
    [128j, 128j+127]; clipped to [0, L))."""
    L = kv.shape[0]
    n = -(-L // r)
    coff = 2 if r == 4 else 1
    out = np.empty((n, 576))
    for j0 in range(0, n, chunk):
        j = np.arange(j0, min(n, j0 + chunk))
        t = (r * j - (coff - 1) * r)[:, None] + np.arange(coff * r)[None, :]
        ok = (t >= 0) & (t < L)
        tc = np.clip(t, 0, L - 1)
        x = kv[tc].astype(np.float64)
        sc = np.where(ok[:, :, None], score[tc].astype(np.float64), -np.inf)
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        den = w.sum(axis=1)
        pooled = (w * x).sum(axis=1) / den
        absum = (w * np.abs(x)).sum(axis=1) / den
        rms = np.sqrt(np.mean(pooled * pooled, axis=1) + eps)
        out[j] = gamma[None, :] * absum / rms[:, None]
    # RoPE mixes each pair (512+2i, 513+2i): either output sums terms of both
    rp = out[:, 512::2] + out[:, 513::2]
    out[:, 512::2] = rp
    out[:, 513::2] = rp
    return out


def near_bf16_midpoint_within(x: np.ndarray, win: np.ndarray) -> np.ndarray:
    """True where the fp32 value x lies within win (absolute) of a bf16
    rounding midpoint (the fp32 patterns ending in 0x8000 around it)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    lower = u & np.uint32(0xFFFF0000)
    mid_hi = (lower | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    mid_lo = np.where(lower & np.uint32(0x7FFF0000), (lower - np.uint32(0x8000)), lower).astype(
        np.uint32).view(np.float32).astype(np.float64)
    a = x.astype(np.float64)
    return np.minimum(np.abs(a - mid_hi), np.abs(a - mid_lo)) <= win


# ------------------------------------------------------------------ oracle side
def oracle_compress(O, lay):
    """Logical slot rows of every sequence, packed by sequence."""
    return O.compress_batch(lay.ratio, lay.cu_seqlens.numpy(), bits16(lay.kv), np_f32(lay.score),
                            np_f32(lay.gamma), lay.eps, np_f32(lay.cos_sin))


def oracle_index_topk(O, lay, queries=None, want_scores=True):
    qs = np.arange(lay.n_q) if queries is None else np.asarray(queries)
    if getattr(lay, "key_fp4", False):
        return O.index_topk_batch_mxfp4(
            lay.k, np_u8(lay.qi)[qs], np_f32(lay.qi_scale)[qs], np_f32(lay.qi_w)[qs],
            np_i32(lay.q_pos)[qs], np_i32(lay.q_seq)[qs], lay.ratio, lay.key_off.numpy(),
            np_i32(lay.n_slots), np_u8(lay.key4_codes), np_u8(lay.key4_e8m0),
            max_slots=lay.max_slots, want_scores=want_scores)
    res = O.index_topk_batch(
        lay.k, np_u8(lay.qi)[qs], np_f32(lay.qi_scale)[qs], np_f32(lay.qi_w)[qs],
        np_i32(lay.q_pos)[qs], np_i32(lay.q_seq)[qs], lay.ratio, lay.key_off.numpy(),
        np_i32(lay.n_slots), np_u8(lay.key_codes), np_f32(lay.key_scales),
        max_slots=lay.max_slots, want_scores=want_scores)
    return res


def oracle_swa_rows(O, lay):
    """The layer's SWA rows as bf16 bits (an fp8 SWA pool: the rows its codes,
    scales and rope stand for)."""
    if getattr(lay, "swa_fp8", False):
        return O.swa_dequant(np_u8(lay.swa_codes), np_f32(lay.swa_scales), bits16(lay.swa_rope))
    return bits16(lay.swa_rows)


def oracle_attention(O, lay, idx, cmp=None, queries=None, want_f64=False):
    """idx: [Q,k] int32 compressed list (None for swaonly).  cmp: dict of logical
    codes/scales/rope (defaults to the layer's given pool contents)."""
    qs = np.arange(lay.n_q) if queries is None else np.asarray(queries)
    swa_rows = oracle_swa_rows(O, lay)
    if lay.ratio > 1 and idx is not None:
        if cmp is None:
            cmp = dict(codes=np_u8(lay.cmp_codes), scales=np_f32(lay.cmp_scales),
                       rope=bits16(lay.cmp_rope))
        return O.sparse_mla_batch(
            bits16(lay.q)[qs], np_i32(lay.q_pos)[qs], np_i32(lay.q_seq)[qs], lay.W,
            lay.swa_off.numpy(), np_i32(lay.swa_base), np_i32(lay.swa_count),
            swa_rows, lay.sm_scale, lay.cmp_off.numpy(), np_i32(lay.n_slots),
            cmp["codes"], cmp["scales"], cmp["rope"], np.ascontiguousarray(idx, np.int32),
            want_f64=want_f64)
    return O.sparse_mla_batch(
        bits16(lay.q)[qs], np_i32(lay.q_pos)[qs], np_i32(lay.q_seq)[qs], lay.W,
        lay.swa_off.numpy(), np_i32(lay.swa_base), np_i32(lay.swa_count), swa_rows,
        lay.sm_scale, want_f64=want_f64)


# --------------------------------------------------------------------- GPU side
def to_device(lay, dev="cuda"):
    """Move every tensor of a Layer to the device (in place) and return it."""
    for name, val in list(vars(lay).items()):
        if isinstance(val, torch.Tensor):
            setattr(lay, name, val.to(dev))
    return lay


def gpu_index_topk(S, lay, scores=True):
    dev = lay.q.device
    ms = lay.max_slots
    sc = torch.full((lay.n_q, ms), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.empty((lay.n_q, lay.k), dtype=torch.int32, device=dev)
    ln = torch.empty(lay.n_q, dtype=torch.int32, device=dev)
    kf = S.KEY_MXFP4 if getattr(lay, "key_fp4", False) else 0
    S.index_scores(lay.qi, lay.qi_scale, lay.qi_w, lay.q_seq, lay.q_pos, lay.ratio | kf,
                   lay.key_pool, lay.key_table, lay.n_slots, ms, sc)
    S.topk_select(lay.k, sc, ms, lay.q_seq, lay.q_pos, lay.ratio, lay.n_slots, idx, ln)
    return sc, idx, ln


def gpu_attention(S, lay, idx, decode=True, cmp_pool=None):
    dev = lay.q.device
    out = torch.empty((lay.n_q, lay.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((lay.n_q, lay.H), dtype=torch.float32, device=dev)
    f = S.sparse_mla_decode if decode else S.sparse_mla_prefill
    fl = S.SWA_FP8 if getattr(lay, "swa_fp8", False) else 0
    if lay.ratio == 1:
        f(1 | fl, lay.q, lay.q_seq, lay.q_pos, lay.W, lay.swa_pool, lay.swa_table,
          sm_scale=lay.sm_scale, out=out, lse=lse)
    else:
        f(lay.ratio | fl, lay.q, lay.q_seq, lay.q_pos, lay.W, lay.swa_pool, lay.swa_table,
          lay.cmp_pool if cmp_pool is None else cmp_pool, lay.cmp_table, idx, lay.n_slots,
          sm_scale=lay.sm_scale, out=out, lse=lse)
    return out, lse


# ----------------------------------------------------------------- acceptance
def check_attention(out_gpu, lse_gpu, out_ref_bits, lse_ref, atol=2e-2, rel=1e-2):
    """bf16 outputs: max |g - o| <= atol and ||g - o|| / ||o|| <= rel; lse abs <= atol."""
    g = out_gpu.float().cpu().numpy().astype(np.float64)
    o = (out_ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(g - o)
    fin = np.isfinite(lse_ref)
    lg = lse_gpu.cpu().numpy()
    assert np.array_equal(np.isfinite(lg), fin), "lse finiteness differs"
    lerr = float(np.max(np.abs(lg[fin] - lse_ref[fin]))) if fin.any() else 0.0
    rl2 = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-30))
    assert err.max() <= atol, f"max abs err {err.max():.3g}"
    assert rl2 <= rel, f"relative L2 err {rl2:.3g}"
    assert lerr <= atol, f"lse err {lerr:.3g}"
    return float(err.max()), rl2, lerr


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """One bf16 step at |x| (8 significant bits): 2^(floor(log2|x|) - 7); 0 at 0."""
    m, e = np.frexp(np.abs(x.astype(np.float64)))
    return np.where(m > 0, np.ldexp(1.0, e - 8), 0.0)


def value_absmax(O, lay, idx):
    """Per query and value dim d: the largest |V_d| over the rows the query
    attends (its window and its valid compressed entries), [Q, 512]."""
    swa = (oracle_swa_rows(O, lay).astype(np.uint32) << 16).view(np.float32)[:, :512]
    qs, qp = np_i32(lay.q_seq), np_i32(lay.q_pos)
    base, off = np_i32(lay.swa_base), lay.swa_off.cpu().numpy()
    ns = np_i32(lay.n_slots)
    out = np.zeros((lay.n_q, 512))
    for t in range(lay.n_q):
        b, p = int(qs[t]), int(qp[t])
        lo = max(0, p - lay.W + 1)
        rows = swa[off[b] + lo - base[b]: off[b] + p - base[b] + 1]
        m = np.abs(rows).max(axis=0) if len(rows) else np.zeros(512)
        if idx is not None and lay.ratio > 1:
            sel = np.asarray(idx[t])
            sel = sel[(sel >= 0) & (sel < ns[b])]
            if len(sel):
                r0 = int(lay.cmp_off[b]) + sel
                v = fp8_values(np_u8(lay.cmp_codes)[r0]) * \
                    np.repeat(np_f32(lay.cmp_scales)[r0].astype(np.float64), 64, axis=1)
                m = np.maximum(m, np.abs(v).max(axis=0))
        out[t] = m
    return out


def check_attention_scaled(out_gpu, lse_gpu, out_ref_bits, lse_ref, vmax, atol=2e-2, rel=1e-2):
    """The attention bar for rows of any dynamic range.  The probabilities
    enter the value product as bf16 (a relative rounding of 2^-9 each), so
    output dim d of a query is off by up to 2^-9 times the weighted mean of
    |V_d|, which is at most vmax[q, d] (value_absmax); the output's own
    rounding to bf16 adds one step at |o|.  Per element:
        |g - o| <= atol + 2^-8 vmax[q, d] + one bf16 step at |o|,
    with the relative L2 error <= rel over all outputs and lse within atol.
    For unit-scale rows (|V| of a few units) this is within 2e-2 of the plain
    bar; it grows only where the rows' values do."""
    g = out_gpu.float().cpu().numpy().astype(np.float64)
    o = (out_ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(g - o)
    fin = np.isfinite(lse_ref)
    lg = lse_gpu.cpu().numpy()
    assert np.array_equal(np.isfinite(lg), fin), "lse finiteness differs"
    lerr = float(np.max(np.abs(lg[fin] - lse_ref[fin]))) if fin.any() else 0.0
    rl2 = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-30))
    bar = atol + 2.0 ** -8 * np.asarray(vmax)[:, None, :] + bf16_ulp(o)
    worst = int(np.argmax(err - bar))
    assert np.all(err <= bar), \
        f"abs err {err.flat[worst]:.3g} above {bar.flat[worst]:.3g} at |o| = {abs(o.flat[worst]):.3g}"
    assert rl2 <= rel, f"relative L2 err {rl2:.3g}"
    assert lerr <= atol, f"lse err {lerr:.3g}"
    return float(err.max()), rl2, lerr, float(np.max(np.abs(o))), float(np.max(vmax))


def check_topk_sets(gpu_idx, gpu_len, ref_scores_rows, nvis, k, rel=1e-6):
    """Per query: the GPU set has min(k, n_vis) distinct entries, contains every
    slot scoring above tau(1+rel) and none below tau(1-rel), tau being the
    oracle's k-th largest score; returns the number of near-tie slots seen."""
    near = 0
    for t in range(gpu_idx.shape[0]):
        n = int(nvis[t])
        kk = min(k, n)
        assert int(gpu_len[t]) == kk
        sel = gpu_idx[t, :kk]
        assert np.all(gpu_idx[t, kk:] == -1)
        assert len(set(sel.tolist())) == kk
        assert np.all((sel >= 0) & (sel < n))
        if kk == n:
            assert set(sel.tolist()) == set(range(n))
            continue
        s = ref_scores_rows[t, :n].astype(np.float64)
        order = np.lexsort((np.arange(n), -s))
        tau = s[order[kk - 1]]
        hi = tau + rel * abs(tau)
        lo = tau - rel * abs(tau)
        must = set(np.nonzero(s > hi)[0].tolist())
        never = set(np.nonzero(s < lo)[0].tolist())
        ss = set(sel.tolist())
        assert must <= ss, f"query {t}: missing {sorted(must - ss)[:5]}"
        assert not (ss & never), f"query {t}: wrongly selected {sorted(ss & never)[:5]}"
        near += int(np.sum((s >= lo) & (s <= hi)))
    return near


def exact_topk_of(scores_rows, nvis, k):
    """Top-k of given fp32 scores with ties to the lower index (numpy lexsort)."""
    out = np.full((scores_rows.shape[0], k), -1, np.int32)
    for t in range(scores_rows.shape[0]):
        n = int(nvis[t])
        s = scores_rows[t, :n].astype(np.float32).astype(np.float64)
        s = np.where(s == 0, 0.0, s)       # -0 == +0
        order = np.lexsort((np.arange(n), -s))[:min(k, n)]
        out[t, :len(order)] = np.sort(order)
    return out
