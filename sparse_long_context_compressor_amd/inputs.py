"""Seeded synthetic inputs for the compressed sparse attention layer.

One module serves both the HIP path and the CPU oracle.  It draws random
tensors and places them into pools; it holds none of the method's arithmetic
(no pooling, normalisation, quantisation rule, scoring, selection or
attention).  fp8 inputs are drawn as torch float8_e4m3fn casts of scaled
normal samples, with independently drawn power-of-two scales.

Recipe (per tensor, each from its own seeded torch.Generator substream):
  queries, SWA rows, per-token kv        N(0,1) -> bf16
  per-token gate scores                  N(0,1) fp32
  compressed rows (given pools)          codes = e4m3(N(0,1)*64), scale 2^U{-8..-5}
                                         per 64 dims, rope N(0,1) -> bf16
  index keys / index queries             codes = e4m3(N(0,1)*64), scale 2^U{-8..-5}
                                         per key / per (query, head)
  head weights                           U(0,1)
  given top-k (c128a)                    the first k of a random permutation of
                                         the slots, per query (distinct, uniform)
  block tables                           a random permutation of the physical
                                         blocks (or the identity when asked)
  RoPE table                             theta = 10000, inv_freq_i = theta^(-2i/64),
                                         angles in float64, stored fp32: 32 cos | 32 sin
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import pools as P

D, DN, DR, DI = P.D_LATENT, P.D_NOPE, P.D_ROPE, P.D_INDEX
BR = P.BLOCK_ROWS


def _gen(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + zlib.crc32(tag.encode())) % (2 ** 62))
    return g


def _randn(shape, seed, tag, device, dtype=torch.float32):
    return torch.randn(shape, generator=_gen(seed, tag, device), device=device,
                       dtype=torch.float32).to(dtype)


def _fp8_codes(shape, seed, tag, device):
    x = torch.randn(shape, generator=_gen(seed, tag, device), device=device) * 64.0
    return x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def _pow2(shape, seed, tag, device, lo=-8, hi=-5):
    e = torch.randint(lo, hi + 1, shape, generator=_gen(seed, tag, device), device=device)
    return torch.pow(2.0, e.to(torch.float32))


def rope_table(max_pos: int, theta: float = 10000.0, device="cpu") -> torch.Tensor:
    i = torch.arange(DR // 2, dtype=torch.float64)
    inv_freq = theta ** (-2.0 * i / DR)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv_freq[None, :]
    return torch.cat([ang.cos(), ang.sin()], dim=1).to(torch.float32).to(device)


def block_table(blocks_needed, width: int, seed: int, tag: str, device, permute=True):
    """blocks_needed: per sequence, the list of logical block ids that hold data.
    Returns (table int32 [n_seq, width] with -1 elsewhere, n_physical_blocks)."""
    total = sum(len(b) for b in blocks_needed)
    phys = (torch.randperm(total, generator=_gen(seed, tag, "cpu")) if permute
            else torch.arange(total))
    table = torch.full((len(blocks_needed), max(width, 1)), -1, dtype=torch.int32)
    k = 0
    for s, blks in enumerate(blocks_needed):
        for lb in blks:
            table[s, lb] = int(phys[k])
            k += 1
    return table.to(device), total


@dataclass
class Layer:
    """Everything one call chain of the layer needs, in logical and pooled form."""
    ratio: int                      # 1 (swaonly), 4 (c4a) or 128 (c128a)
    n_seq: int
    H: int
    W: int
    k: int
    H_I: int
    sm_scale: float
    q: torch.Tensor                 # [Q,H,576] bf16
    q_seq: torch.Tensor             # [Q] int32
    q_pos: torch.Tensor             # [Q] int32
    swa_base: torch.Tensor          # [n_seq] int32: first position with a SWA row
    swa_count: torch.Tensor         # [n_seq] int32
    swa_rows: Optional[torch.Tensor]  # [sum counts, 576] bf16, sequences back to back
    swa_off: torch.Tensor           # [n_seq] int64 row offsets into swa_rows
    swa_pool: torch.Tensor
    swa_table: torch.Tensor
    n_slots: torch.Tensor           # [n_seq] int32 (0 for swaonly)
    cmp_table: Optional[torch.Tensor] = None
    cmp_pool: Optional[torch.Tensor] = None
    cmp_off: Optional[torch.Tensor] = None     # [n_seq] int64
    cmp_codes: Optional[torch.Tensor] = None   # [sum slots, 512] uint8
    cmp_scales: Optional[torch.Tensor] = None  # [sum slots, 8] f32
    cmp_rope: Optional[torch.Tensor] = None    # [sum slots, 64] bf16
    key_table: Optional[torch.Tensor] = None
    key_pool: Optional[torch.Tensor] = None
    key_off: Optional[torch.Tensor] = None
    key_codes: Optional[torch.Tensor] = None   # [sum slots, 128] uint8
    key_scales: Optional[torch.Tensor] = None  # [sum slots] f32
    qi: Optional[torch.Tensor] = None          # [Q,H_I,128] uint8
    qi_scale: Optional[torch.Tensor] = None    # [Q,H_I] f32
    qi_w: Optional[torch.Tensor] = None        # [Q,H_I] f32
    given_idx: Optional[torch.Tensor] = None   # [Q,k] int32 (c128a)
    # compress inputs (only when the compressed rows are to be produced by compress)
    cu_seqlens: Optional[torch.Tensor] = None
    kv: Optional[torch.Tensor] = None          # [T,576] bf16
    score: Optional[torch.Tensor] = None       # [T,576] f32
    gamma: Optional[torch.Tensor] = None
    eps: float = 1e-6
    cos_sin: Optional[torch.Tensor] = None
    cmp_blocks: int = 0
    # fp8 SWA pool (compressed-row layout) instead of bf16 rows
    swa_fp8: bool = False
    swa_codes: Optional[torch.Tensor] = None   # [sum counts, 512] uint8
    swa_scales: Optional[torch.Tensor] = None  # [sum counts, 8] f32
    swa_rope: Optional[torch.Tensor] = None    # [sum counts, 64] bf16
    # MXFP4 index keys (key_pool then has the KEY4 layout)
    key_fp4: bool = False
    key4_codes: Optional[torch.Tensor] = None  # [sum slots, 64] uint8
    key4_e8m0: Optional[torch.Tensor] = None   # [sum slots, 4] uint8
    extra: dict = field(default_factory=dict)

    @property
    def n_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_slots(self) -> int:
        return int(self.n_slots.max()) if self.n_slots.numel() else 0


def build_layer(seed: int, *, ratio: int, H: int, ctx: list, queries: list, n_slots: list,
                W: int = 128, k: int = 0, H_I: int = 0, given_topk: bool = False,
                permute: bool = True, compress_inputs: bool = False, swa_fp8: bool = False,
                key_fp4: bool = False, swa_scale_exp: tuple = (-6, -6),
                gamma_random: bool = False, sm_scale: Optional[float] = None,
                device="cpu") -> Layer:
    """ctx[b]: context length of sequence b; queries: list of (seq, position);
    n_slots[b]: compressed slots of sequence b (stated by the caller).
    SWA rows are drawn for positions [min_q max(0, p-W+1), max_q p] per sequence.
    swa_scale_exp: with swa_fp8, each 64-dim block of an SWA row takes the scale
    2^e, e uniform on [lo, hi] (the default (-6, -6) gives unit-scale rows)."""
    n_seq = len(ctx)
    dev = device
    q_seq = torch.tensor([s for s, _ in queries], dtype=torch.int32)
    q_pos = torch.tensor([p for _, p in queries], dtype=torch.int32)
    Q = len(queries)
    q = _randn((Q, H, D), seed, "q", dev, torch.bfloat16)

    # ---- per-token kv/score (compress inputs) ----------------------------
    cu = torch.zeros(n_seq + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(ctx, dtype=torch.int32), 0)
    kv = score = gamma = cos_sin = None
    if compress_inputs:
        T = int(cu[-1])
        kv = _randn((T, D), seed, "kv", dev, torch.bfloat16)
        score = _randn((T, D), seed, "score", dev)
        gamma = (_randn((D,), seed, "gamma", dev).abs() + 0.5) if gamma_random else \
            torch.ones(D, dtype=torch.float32, device=dev)
        cos_sin = rope_table(max(ctx), device=dev)

    # ---- SWA rows and pool ------------------------------------------------
    swa_base, swa_count = [], []
    for b in range(n_seq):
        ps = [p for s, p in queries if s == b]
        lo = max(0, min(ps) - W + 1) if ps else 0
        hi = max(ps) if ps else -1
        swa_base.append(lo)
        swa_count.append(hi - lo + 1)
    rows, offs = [], []
    off = 0
    for b in range(n_seq):
        offs.append(off)
        if compress_inputs:
            t0 = int(cu[b])
            rows.append(kv[t0 + swa_base[b]: t0 + swa_base[b] + swa_count[b]].to(torch.bfloat16))
        else:
            rows.append(_randn((swa_count[b], D), seed, f"swa{b}", dev, torch.bfloat16))
        off += swa_count[b]
    swa_rows = torch.cat(rows, 0) if rows else torch.zeros(0, D, dtype=torch.bfloat16, device=dev)
    swa_blocks = [list(range(swa_base[b] // BR, (swa_base[b] + swa_count[b] - 1) // BR + 1))
                  if swa_count[b] > 0 else [] for b in range(n_seq)]
    width = max(1, -(-max(ctx) // BR))
    swa_table, nsb = block_table(swa_blocks, width, seed, "swa_table", dev, permute)
    swa_codes = swa_scales = swa_rope = None
    if swa_fp8:
        # fp8 SWA rows in the compressed-row layout: random codes (N(0, 64)
        # before the e4m3 cast) with per-block scales 2^U{lo..hi} (by default
        # 2^-6, so that the rows are unit-scale like the bf16 SWA rows), and
        # bf16 rope dims (swa_rows is then left unset)
        nrow = swa_rows.shape[0]
        swa_codes = _fp8_codes((nrow, DN), seed, "swa_codes", dev)
        swa_scales = _pow2((nrow, DN // 64), seed, "swa_scales", dev, lo=swa_scale_exp[0],
                           hi=swa_scale_exp[1])
        swa_rope = _randn((nrow, DR), seed, "swa_rope", dev, torch.bfloat16)
        swa_rows = None
        swa_pool = P.cmp_pool_empty(nsb, dev)
        for b in range(n_seq):
            if swa_count[b] > 0:
                sl = slice(offs[b], offs[b] + swa_count[b])
                P.cmp_pool_put(swa_pool, swa_table[b], swa_base[b], swa_codes[sl],
                               swa_scales[sl], swa_rope[sl])
    else:
        swa_pool = P.swa_pool_empty(nsb, dev)
        for b in range(n_seq):
            if swa_count[b] > 0:
                P.swa_pool_put(swa_pool, swa_table[b], swa_base[b],
                               swa_rows[offs[b]: offs[b] + swa_count[b]])

    lay = Layer(ratio=ratio, n_seq=n_seq, H=H, W=W, k=k, H_I=H_I,
                sm_scale=(1.0 / math.sqrt(D)) if sm_scale is None else sm_scale,
                q=q, q_seq=q_seq.to(dev), q_pos=q_pos.to(dev),
                swa_base=torch.tensor(swa_base, dtype=torch.int32, device=dev),
                swa_count=torch.tensor(swa_count, dtype=torch.int32, device=dev),
                swa_rows=swa_rows, swa_off=torch.tensor(offs, dtype=torch.int64, device=dev),
                swa_pool=swa_pool, swa_table=swa_table,
                n_slots=torch.tensor(n_slots if ratio > 1 else [0] * n_seq, dtype=torch.int32,
                                     device=dev),
                cu_seqlens=cu.to(dev), kv=kv, score=score, gamma=gamma, cos_sin=cos_sin,
                swa_fp8=swa_fp8, swa_codes=swa_codes, swa_scales=swa_scales,
                swa_rope=swa_rope)
    if ratio <= 1:
        return lay

    # ---- compressed pool ----------------------------------------------------
    cmp_off = [0] * n_seq
    tot = 0
    for b in range(n_seq):
        cmp_off[b] = tot
        tot += n_slots[b]
    cblocks = [list(range(-(-n_slots[b] // BR))) for b in range(n_seq)]
    cwidth = max(1, max((-(-n // BR)) for n in n_slots))
    cmp_table, ncb = block_table(cblocks, cwidth, seed, "cmp_table", dev, permute)
    lay.cmp_table = cmp_table
    lay.cmp_blocks = ncb
    lay.cmp_pool = P.cmp_pool_empty(ncb, dev)
    lay.cmp_off = torch.tensor(cmp_off, dtype=torch.int64, device=dev)
    if not compress_inputs:
        codes = _fp8_codes((tot, DN), seed, "cmp_codes", dev)
        scales = _pow2((tot, DN // 64), seed, "cmp_scales", dev)
        rope = _randn((tot, DR), seed, "cmp_rope", dev, torch.bfloat16)
        lay.cmp_codes, lay.cmp_scales, lay.cmp_rope = codes, scales, rope
        for b in range(n_seq):
            s0, n = cmp_off[b], n_slots[b]
            if n:
                P.cmp_pool_put(lay.cmp_pool, cmp_table[b], 0, codes[s0:s0 + n],
                               scales[s0:s0 + n], rope[s0:s0 + n])

    # ---- indexer (c4a) --------------------------------------------------------
    if ratio == 4 and H_I > 0:
        kcodes = _fp8_codes((tot, DI), seed, "key_codes", dev)
        kscales = _pow2((tot,), seed, "key_scales", dev)
        key_table, nkb = block_table(cblocks, cwidth, seed, "key_table", dev, permute)
        key_pool = P.key_pool_empty(nkb, dev)
        for b in range(n_seq):
            s0, n = cmp_off[b], n_slots[b]
            if n:
                P.key_pool_put(key_pool, key_table[b], 0, kcodes[s0:s0 + n], kscales[s0:s0 + n])
        lay.key_table, lay.key_pool = key_table, key_pool
        lay.key_off = lay.cmp_off.clone()
        lay.key_codes, lay.key_scales = kcodes, kscales
        if key_fp4:
            # MXFP4 keys instead: random e2m1 pairs and E8M0 block scales
            g4 = _gen(seed, "key4", "cpu")
            lay.key4_codes = torch.randint(0, 256, (tot, DI // 2), generator=g4,
                                           dtype=torch.uint8).to(dev)
            lay.key4_e8m0 = torch.randint(120, 131, (tot, DI // 32), generator=g4,
                                          dtype=torch.uint8).to(dev)
            lay.key_fp4 = True
            lay.key_pool = P.key4_pool_empty(nkb, dev)
            for b in range(n_seq):
                s0, n = cmp_off[b], n_slots[b]
                if n:
                    P.key4_pool_put(lay.key_pool, key_table[b], 0, lay.key4_codes[s0:s0 + n],
                                    lay.key4_e8m0[s0:s0 + n])
        lay.qi = _fp8_codes((Q, H_I, DI), seed, "qi", dev)
        lay.qi_scale = _pow2((Q, H_I), seed, "qi_scale", dev)
        lay.qi_w = torch.rand((Q, H_I), generator=_gen(seed, "qi_w", dev), device=dev)

    # ---- given top-k (c128a) ----------------------------------------------
    if given_topk and k > 0:
        idx = torch.full((Q, k), -1, dtype=torch.int32)
        g = _gen(seed, "given_idx", "cpu")
        for t, (s, _) in enumerate(queries):
            perm = torch.randperm(n_slots[s], generator=g)[:k]
            idx[t, :perm.numel()] = perm.to(torch.int32)
        lay.given_idx = idx.to(dev)
    return lay


# ------------------------------------------------------------------ configs
# The five workloads, named by what they are.  Sizes as stated for each.
def c4a_single_layer_4k(seed=0, device="cpu") -> Layer:
    """C4A single-layer decode, batch 1, H=16, context 4096 compressed (r=4,
    8-token overlapping gather) into 1024 slots, SWA 128, indexer 16 heads,
    top-k 256, sm_scale 1/sqrt(576)."""
    return build_layer(seed, ratio=4, H=16, ctx=[4096], queries=[(0, 4095)], n_slots=[1024],
                       W=128, k=256, H_I=16, compress_inputs=True, device=device)


def swaonly_decode_b64(seed=1, device="cpu", swa_fp8=False) -> Layer:
    """swaonly decode, batch 64, H=64, context 8192, only the last 128 tokens
    attended; blocks laid out contiguously (swa_fp8: an fp8 SWA pool)."""
    return build_layer(seed, ratio=1, H=64, ctx=[8192] * 64,
                       queries=[(b, 8191) for b in range(64)], n_slots=[0] * 64, W=128,
                       permute=False, swa_fp8=swa_fp8, device=device)


def c4a_decode_64k(seed=2, device="cpu", batch=32, swa_fp8=False, key_fp4=False) -> Layer:
    """C4A decode, batch 32, H=64, context 65536 -> 16384 slots per sequence,
    indexer 64 heads x 128, top-k 512 + SWA 128, 64-row blocks, permuted tables
    (swa_fp8: the SWA pool holds fp8 rows in the compressed-row layout;
    key_fp4: the index keys are MXFP4)."""
    return build_layer(seed, ratio=4, H=64, ctx=[65536] * batch,
                       queries=[(b, 65535) for b in range(batch)], n_slots=[16384] * batch,
                       W=128, k=512, H_I=64, swa_fp8=swa_fp8, key_fp4=key_fp4, device=device)


def c128a_decode_128k(seed=3, device="cpu", batch=32, swa_fp8=False) -> Layer:
    """C128A decode, batch 32, H=64, context 131072 -> 1024 slots, given top-k
    512 distinct uniform samples per query, SWA 128 (swa_fp8: an fp8 SWA pool)."""
    return build_layer(seed, ratio=128, H=64, ctx=[131072] * batch,
                       queries=[(b, 131071) for b in range(batch)], n_slots=[1024] * batch,
                       W=128, k=512, given_topk=True, swa_fp8=swa_fp8, device=device)


def c4a_prefill_2k(seed=4, device="cpu", swa_fp8=False, key_fp4=False) -> Layer:
    """C4A prefill chunk: 2048 causal query tokens at positions 129024..131071,
    H=64, context 131072 -> 32768 slots, indexer 64 heads, top-k 2048 + SWA 128
    (swa_fp8 / key_fp4: the fp8 SWA pool and MXFP4 index keys)."""
    return build_layer(seed, ratio=4, H=64, ctx=[131072],
                       queries=[(0, p) for p in range(129024, 131072)], n_slots=[32768],
                       W=128, k=2048, H_I=64, swa_fp8=swa_fp8, key_fp4=key_fp4, device=device)


CONFIGS = {
    "c4a_single_layer_4k": c4a_single_layer_4k,
    "swaonly_decode_b64": swaonly_decode_b64,
    "c4a_decode_64k": c4a_decode_64k,
    "c128a_decode_128k": c128a_decode_128k,
    "c4a_prefill_2k": c4a_prefill_2k,
}
