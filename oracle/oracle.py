"""ctypes wrapper over liboracle_slc.so (built from slc_oracle.c with gcc).

TEST INFRASTRUCTURE ONLY.  Arrays are numpy, host memory, logical layout
(one row per token / slot, no paging).  bf16 values travel as their uint16
bit patterns and e4m3 values as uint8 codes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

__all__ = [
    "build", "lib", "e4m3_decode", "e4m3_encode", "bf16_decode", "bf16_encode",
    "pow2_scale", "n_slots", "n_visible", "window", "compress_seq", "compress_batch",
    "compress_stream_seq", "compress_index_keys_stream_seq",
    "index_scores", "topk", "index_topk_batch", "sparse_mla", "sparse_mla_batch",
    "swa_insert", "swa_dequant", "e2m1_value", "e8m0_value", "mxfp4_quantise", "index_scores_mxfp4",
    "index_topk_batch_mxfp4", "indexcache_skips", "num_threads",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "slc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_slc.so")
_lib = None

D, DN, DR, QB, DI = 576, 512, 64, 64, 128


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11 + OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-std=gnu11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
             "-shared", "-o", tmp, _SRC, "-lm"],
            check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = C.c_void_p


def _declare(L):
    i32, i64, dbl = C.c_int, C.c_int64, C.c_double
    sig = {
        "oracle_e4m3_value": (dbl, [C.c_uint8]),
        "oracle_e4m3_encode": (C.c_uint8, [dbl]),
        "oracle_bf16_value": (dbl, [C.c_uint16]),
        "oracle_bf16_encode": (C.c_uint16, [dbl]),
        "oracle_pow2_scale": (dbl, [dbl]),
        "oracle_n_slots": (i32, [i32, i32]),
        "oracle_n_visible": (i32, [i32, i32, i32]),
        "oracle_window": (None, [i32, i32, i32, _P, _P]),
        "oracle_compress_seq": (i32, [i32, i32, _P, _P, _P, dbl, _P, i32, _P, _P, _P, _P, _P]),
        "oracle_compress_batch": (i32, [i32, i32, _P, _P, _P, _P, dbl, _P, i32, _P, _P, _P, _P]),
        "oracle_index_scores": (None, [i32, i32, _P, _P, _P, _P, _P, _P, _P]),
        "oracle_topk": (i32, [i32, _P, i32, _P]),
        "oracle_index_topk_batch": (None, [i32, i32, i32, _P, _P, _P, _P, _P, i32, _P, _P,
                                           _P, _P, _P, _P, _P, i32]),
        "oracle_sparse_mla": (i32, [i32, _P, i32, i32, i32, i32, _P, i32, _P, _P, _P, i32, _P,
                                    dbl, _P, _P, _P, _P]),
        "oracle_sparse_mla_batch": (i32, [i32, i32, _P, _P, _P, i32, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _P, i32, _P, dbl, _P, _P, _P, _P]),
        "oracle_swa_insert": (i32, [i32, _P, _P, _P, i32, _P, _P, _P, _P]),
        "oracle_compress_index_keys_stream_seq": (i32, [i32, _P, _P, _P, _P, dbl, _P, i32, _P,
                                                        _P, _P]),
        "oracle_compress_stream_seq": (i32, [i32, i32, _P, _P, _P, _P, dbl, _P, i32, _P, _P, _P,
                                             _P]),
        "oracle_e2m1_value": (dbl, [C.c_uint8]),
        "oracle_mxfp4_quantise": (None, [i32, _P, _P, _P]),
        "oracle_e8m0_value": (dbl, [C.c_uint8]),
        "oracle_index_scores_mxfp4": (None, [i32, i32, _P, _P, _P, _P, _P, _P, _P]),
        "oracle_index_topk_batch_mxfp4": (None, [i32, i32, i32, _P, _P, _P, _P, _P, i32, _P,
                                                 _P, _P, _P, _P, _P, _P, i32]),
        "oracle_num_threads": (i32, []),
        "oracle_e4m3_decode_array": (None, [i64, _P, _P]),
        "oracle_e4m3_encode_array": (None, [i64, _P, _P]),
        "oracle_bf16_decode_array": (None, [i64, _P, _P]),
        "oracle_bf16_encode_array": (None, [i64, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _c(a, dtype):
    """Contiguous numpy array of the exact dtype (no silent value conversion
    for integer bit patterns: uint8 / uint16 inputs must already be those)."""
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        if np.dtype(dtype).kind in "iu" and a.dtype.kind == "f":
            raise TypeError(f"expected {dtype} bit patterns, got {a.dtype}")
        a = a.astype(dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


# ------------------------------------------------------------------ codecs
def e4m3_decode(codes):
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_array(c.size, _p(c), _p(out))
    return out


def e4m3_encode(x):
    v = _c(x, np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_encode_array(v.size, _p(v), _p(out))
    return out


def bf16_decode(bits):
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().oracle_bf16_decode_array(b.size, _p(b), _p(out))
    return out


def bf16_encode(x):
    v = _c(x, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_encode_array(v.size, _p(v), _p(out))
    return out


def pow2_scale(amax: float) -> float:
    return lib().oracle_pow2_scale(float(amax))


# ------------------------------------------------------------ slot algebra
def n_slots(L: int, r: int) -> int:
    return lib().oracle_n_slots(L, r)


def n_visible(p: int, r: int, ns: int) -> int:
    return lib().oracle_n_visible(p, r, ns)


def window(j: int, r: int, L: int):
    lo, hi = C.c_int(), C.c_int()
    lib().oracle_window(j, r, L, C.byref(lo), C.byref(hi))
    return lo.value, hi.value


# ---------------------------------------------------------------- compress
def compress_seq(r, kv_bits, score, gamma, eps, cos_sin):
    """One sequence.  Returns dict(codes [n,512] u8, scales [n,8] f32,
    rope [n,64] u16, pooled [n,576] f64, prequant [n,576] f32)."""
    kv = _c(kv_bits, np.uint16)
    sc = _c(score, np.float32)
    g = _c(gamma, np.float32)
    cs = _c(cos_sin, np.float32)
    L = kv.shape[0]
    n = n_slots(L, r)
    codes = np.zeros((n, DN), np.uint8)
    scales = np.zeros((n, DN // QB), np.float32)
    rope = np.zeros((n, DR), np.uint16)
    pooled = np.zeros((n, D), np.float64)
    pre = np.zeros((n, D), np.float32)
    rc = lib().oracle_compress_seq(r, L, _p(kv), _p(sc), _p(g), float(eps), _p(cs), cs.shape[0],
                                   _p(codes), _p(scales), _p(rope), _p(pooled), _p(pre))
    if rc:
        raise ValueError("slot anchor position outside the cos/sin table")
    return dict(codes=codes, scales=scales, rope=rope, pooled=pooled, prequant=pre)


def compress_stream_seq(r, kv_bits, score, ape, gamma, eps, cos_sin):
    """Streaming (two-block) compressor over one sequence's L tokens: kv
    [L, coff*576] bf16 bits, score [L, coff*576] f32, ape [r, coff*576] f32.
    Returns dict(codes, scales, rope, prequant) for the floor(L/r) slots."""
    coff = 2 if r == 4 else 1
    kv = _c(kv_bits, np.uint16).reshape(-1, coff * D)
    L = kv.shape[0]
    sc = _c(score, np.float32).reshape(L, coff * D)
    ap = _c(ape, np.float32).reshape(r, coff * D)
    g = _c(gamma, np.float32)
    cs = _c(cos_sin, np.float32)
    n = L // r
    codes = np.zeros((n, DN), np.uint8)
    scales = np.zeros((n, DN // QB), np.float32)
    rope = np.zeros((n, DR), np.uint16)
    pre = np.zeros((n, D), np.float32)
    if lib().oracle_compress_stream_seq(r, L, _p(kv), _p(sc), _p(ap), _p(g), float(eps), _p(cs),
                                        cs.shape[0], _p(codes), _p(scales), _p(rope), _p(pre)):
        raise ValueError("slot anchor position outside the cos/sin table")
    return dict(codes=codes, scales=scales, rope=rope, prequant=pre)


def compress_index_keys_stream_seq(kv_bits, score, ape, gamma, eps, cos_sin):
    """The indexer's 128-dim key compressor (ratio 4, two blocks) over one
    sequence: kv [L, 256] bf16 bits, score [L, 256], ape [4, 256], gamma [128].
    Returns dict(codes [n,128], scales [n], prequant [n,128]), n = L // 4."""
    kv = _c(kv_bits, np.uint16).reshape(-1, 2 * DI)
    L = kv.shape[0]
    sc = _c(score, np.float32).reshape(L, 2 * DI)
    ap = _c(ape, np.float32).reshape(4, 2 * DI)
    g = _c(gamma, np.float32)
    cs = _c(cos_sin, np.float32)
    n = L // 4
    codes = np.zeros((n, DI), np.uint8)
    scales = np.zeros(n, np.float32)
    pre = np.zeros((n, DI), np.float32)
    if lib().oracle_compress_index_keys_stream_seq(L, _p(kv), _p(sc), _p(ap), _p(g), float(eps),
                                                   _p(cs), cs.shape[0], _p(codes), _p(scales),
                                                   _p(pre)):
        raise ValueError("slot anchor position outside the cos/sin table")
    return dict(codes=codes, scales=scales, prequant=pre)


def compress_batch(r, cu_seqlens, kv_bits, score, gamma, eps, cos_sin):
    """Sequences packed by cu_seqlens; slot outputs packed in the same order."""
    cu = _c(cu_seqlens, np.int32)
    kv = _c(kv_bits, np.uint16)
    sc = _c(score, np.float32)
    g = _c(gamma, np.float32)
    cs = _c(cos_sin, np.float32)
    tot = sum(n_slots(int(cu[b + 1] - cu[b]), r) for b in range(len(cu) - 1))
    codes = np.zeros((tot, DN), np.uint8)
    scales = np.zeros((tot, DN // QB), np.float32)
    rope = np.zeros((tot, DR), np.uint16)
    pre = np.zeros((tot, D), np.float32)
    rc = lib().oracle_compress_batch(r, len(cu) - 1, _p(cu), _p(kv), _p(sc), _p(g), float(eps),
                                     _p(cs), cs.shape[0], _p(codes), _p(scales), _p(rope), _p(pre))
    if rc:
        raise ValueError("slot anchor position outside the cos/sin table")
    return dict(codes=codes, scales=scales, rope=rope, prequant=pre)


# ----------------------------------------------------------------- indexer
def index_scores(q_codes, q_scale, w, key_codes, key_scale):
    """One query: q [H_I,128] u8, q_scale/w [H_I], keys [n,128] u8, key_scale [n].
    Returns (fp32 scores [n], float64 scores [n])."""
    q = _c(q_codes, np.uint8)
    qs = _c(q_scale, np.float32)
    ww = _c(w, np.float32)
    k = _c(key_codes, np.uint8)
    ks = _c(key_scale, np.float32)
    n = k.shape[0]
    s32 = np.zeros(n, np.float32)
    s64 = np.zeros(n, np.float64)
    lib().oracle_index_scores(q.shape[0], n, _p(q), _p(qs), _p(ww), _p(k), _p(ks), _p(s32), _p(s64))
    return s32, s64


def topk(scores32, k):
    s = _c(scores32, np.float32)
    idx = np.zeros(k, np.int32)
    ln = lib().oracle_topk(s.shape[0], _p(s), k, _p(idx))
    return idx, ln


def index_topk_batch(k, q_codes, q_scale, w, q_pos, q_seq, r, key_off, n_slots_,
                     key_codes, key_scale, max_slots=None, want_scores=False):
    q = _c(q_codes, np.uint8)
    nq, hI = q.shape[0], q.shape[1]
    qs = _c(q_scale, np.float32)
    ww = _c(w, np.float32)
    qp = _c(q_pos, np.int32)
    qsq = _c(q_seq, np.int32)
    ko = _c(key_off, np.int64)
    ns = _c(n_slots_, np.int32)
    kc = _c(key_codes, np.uint8)
    ksc = _c(key_scale, np.float32)
    idx = np.zeros((nq, k), np.int32)
    ln = np.zeros(nq, np.int32)
    ms = int(max_slots if max_slots is not None else (ns.max() if ns.size else 0))
    sc = np.full((nq, ms), np.nan, np.float32) if want_scores else None
    lib().oracle_index_topk_batch(nq, hI, k, _p(q), _p(qs), _p(ww), _p(qp), _p(qsq), r, _p(ko),
                                  _p(ns), _p(kc), _p(ksc), _p(idx), _p(ln), _p(sc), ms)
    return (idx, ln, sc) if want_scores else (idx, ln)


def e2m1_value(nibble: int) -> float:
    return lib().oracle_e2m1_value(int(nibble))


def e8m0_value(b: int) -> float:
    return lib().oracle_e8m0_value(int(b))


def mxfp4_quantise(y):
    """y [n,128] f32 -> (codes4 [n,64] u8, e8m0 [n,4] u8): per 32-dim block the
    smallest 2^e with amax <= 6 * 2^e, nearest e2m1 codes (ties to even)."""
    v = _c(y, np.float32).reshape(-1, DI)
    n = v.shape[0]
    c4 = np.zeros((n, DI // 2), np.uint8)
    e8 = np.zeros((n, DI // 32), np.uint8)
    lib().oracle_mxfp4_quantise(n, _p(v), _p(c4), _p(e8))
    return c4, e8


def index_scores_mxfp4(q_codes, q_scale, w, keys4, key_e8m0):
    """One query against MXFP4 keys: keys4 [n,64] u8 (two e2m1 per byte, even
    element low), key_e8m0 [n,4] u8.  Returns (fp32 scores [n], float64 [n])."""
    q = _c(q_codes, np.uint8)
    qs = _c(q_scale, np.float32)
    ww = _c(w, np.float32)
    k = _c(keys4, np.uint8)
    ke = _c(key_e8m0, np.uint8)
    n = k.shape[0]
    s32 = np.zeros(n, np.float32)
    s64 = np.zeros(n, np.float64)
    lib().oracle_index_scores_mxfp4(q.shape[0], n, _p(q), _p(qs), _p(ww), _p(k), _p(ke), _p(s32),
                                    _p(s64))
    return s32, s64


def index_topk_batch_mxfp4(k, q_codes, q_scale, w, q_pos, q_seq, r, key_off, n_slots_,
                           keys4, key_e8m0, max_slots=None, want_scores=False):
    q = _c(q_codes, np.uint8)
    nq, hI = q.shape[0], q.shape[1]
    ns = _c(n_slots_, np.int32)
    idx = np.zeros((nq, k), np.int32)
    ln = np.zeros(nq, np.int32)
    ms = int(max_slots if max_slots is not None else (ns.max() if ns.size else 0))
    sc = np.full((nq, ms), np.nan, np.float32) if want_scores else None
    args = [_c(q_scale, np.float32), _c(w, np.float32), _c(q_pos, np.int32),
            _c(q_seq, np.int32)]
    ko = _c(key_off, np.int64)
    k4 = _c(keys4, np.uint8)
    ke = _c(key_e8m0, np.uint8)
    lib().oracle_index_topk_batch_mxfp4(nq, hI, k, _p(q), *map(_p, args), r, _p(ko), _p(ns),
                                        _p(k4), _p(ke), _p(idx), _p(ln), _p(sc), ms)
    return (idx, ln, sc) if want_scores else (idx, ln)


# --------------------------------------------------------------- attention
def sparse_mla(q_bits, p, W, swa_base, swa_rows, sm_scale, codes=None, scales=None,
               rope=None, idx=None):
    """One query: q [H,576] u16.  Returns (out u16 [H,512], lse f32 [H],
    out f64 [H,512], lse f64 [H])."""
    q = _c(q_bits, np.uint16)
    h = q.shape[0]
    sw = _c(swa_rows, np.uint16)
    if idx is None:
        k, ns, cd, scl, rp, ix = 0, 0, None, None, None, None
    else:
        ix = _c(idx, np.int32)
        k = ix.shape[0]
        cd = _c(codes, np.uint8)
        scl = _c(scales, np.float32)
        rp = _c(rope, np.uint16)
        ns = cd.shape[0]
    out = np.zeros((h, DN), np.uint16)
    lse = np.zeros(h, np.float32)
    o64 = np.zeros((h, DN), np.float64)
    l64 = np.zeros(h, np.float64)
    rc = lib().oracle_sparse_mla(h, _p(q), int(p), int(W), int(swa_base), sw.shape[0], _p(sw), ns,
                                 _p(cd), _p(scl), _p(rp), k, _p(ix), float(sm_scale), _p(out),
                                 _p(lse), _p(o64), _p(l64))
    if rc:
        raise ValueError("SWA rows do not cover the query's window")
    return out, lse, o64, l64


def sparse_mla_batch(q_bits, q_pos, q_seq, W, swa_off, swa_base, swa_count, swa_rows,
                     sm_scale, cmp_off=None, n_slots_=None, codes=None, scales=None,
                     rope=None, idx=None, want_f64=False):
    q = _c(q_bits, np.uint16)
    nq, h = q.shape[0], q.shape[1]
    qp = _c(q_pos, np.int32)
    qsq = _c(q_seq, np.int32)
    so = _c(swa_off, np.int64)
    sb = _c(swa_base, np.int32)
    scn = _c(swa_count, np.int32)
    sw = _c(swa_rows, np.uint16)
    if idx is None:
        k, co, ns, cd, scl, rp, ix = 0, None, None, None, None, None, None
    else:
        ix = _c(idx, np.int32)
        k = ix.shape[1]
        co = _c(cmp_off, np.int64)
        ns = _c(n_slots_, np.int32)
        cd = _c(codes, np.uint8)
        scl = _c(scales, np.float32)
        rp = _c(rope, np.uint16)
    out = np.zeros((nq, h, DN), np.uint16)
    lse = np.zeros((nq, h), np.float32)
    o64 = np.zeros((nq, h, DN), np.float64) if want_f64 else None
    l64 = np.zeros((nq, h), np.float64) if want_f64 else None
    rc = lib().oracle_sparse_mla_batch(nq, h, _p(q), _p(qp), _p(qsq), int(W), _p(so), _p(sb),
                                       _p(scn), _p(sw), _p(co), _p(ns), _p(cd), _p(scl), _p(rp),
                                       k, _p(ix), float(sm_scale), _p(out), _p(lse), _p(o64),
                                       _p(l64))
    if rc:
        raise ValueError("SWA rows do not cover some query's window")
    if want_f64:
        return out, lse, o64, l64
    return out, lse


# --------------------------------------------------------- FP8 SWA rows
def swa_insert(kv_bits, pos, cos_sin):
    """SWA KV insert of n tokens (kv [n,576] bf16 bits, not yet rotated; pos
    [n] their positions): RoPE at each token's own position, then the cache
    row format.  Returns codes u8 [n,512], scales f32 [n,8], rope u16 [n,64]
    and the fp32 rows before quantisation [n,576]."""
    kv = _c(kv_bits, np.uint16).reshape(-1, D)
    n = kv.shape[0]
    ps = _c(pos, np.int32)
    cs = _c(cos_sin, np.float32)
    codes = np.zeros((n, DN), np.uint8)
    scales = np.zeros((n, DN // 64), np.float32)
    rope = np.zeros((n, DR), np.uint16)
    pre = np.zeros((n, D), np.float32)
    if lib().oracle_swa_insert(n, _p(kv), _p(ps), _p(cs), cs.shape[0], _p(codes), _p(scales),
                               _p(rope), _p(pre)):
        raise ValueError("a position is outside the cos/sin table")
    return codes, scales, rope, pre


def swa_dequant(codes, scales, rope):
    """The latent rows an fp8 cache row stands for, as bf16 bits [n,576]:
    code * scale for the nope dims (exact in bf16 for power-of-two scales,
    which is checked), the rope dims as stored."""
    cd = _c(codes, np.uint8)
    n = cd.shape[0]
    v = e4m3_decode(cd) * np.repeat(_c(scales, np.float32).astype(np.float64), 64, axis=1)
    nope = bf16_encode(v)
    if not np.array_equal(bf16_decode(nope), v):
        raise ValueError("code * scale is not exact in bf16")
    return np.concatenate([nope, _c(rope, np.uint16).reshape(n, DR)], axis=1)


# ------------------------------------------------------------- IndexCache
def indexcache_skips(compress_ratios, freq: int, pattern: str = ""):
    """Per layer: 1 if the layer reuses an earlier layer's top-k, else 0.

    "DeepSeek-V4 IndexCache freq2 cross-layer TopK reuse" page, section 2:
    only layers with compress ratio 4 take part; a layer's indexer sequence
    index is the number of ratio-4 layers before it; without a pattern the
    layer reuses when that index is not a multiple of the frequency; a
    pattern string, when given, takes priority: it must begin with 'F'
    (compute), 'S' at the layer's sequence index means reuse, and layers past
    the end of the string compute.  A frequency of 1 (or less) never reuses.
    """
    if pattern and pattern[0] != "F":
        raise ValueError("an IndexCache pattern must begin with 'F'")
    if pattern and any(ch not in "FS" for ch in pattern):
        raise ValueError("an IndexCache pattern holds only 'F' and 'S'")
    out = []
    seq = 0                                   # ratio-4 layers seen before this one
    for r in compress_ratios:
        if r != 4:
            out.append(0)
            continue
        if pattern:
            skip = seq < len(pattern) and pattern[seq] == "S"
        else:
            skip = freq > 1 and seq % freq != 0
        out.append(1 if skip else 0)
        seq += 1
    return out


def num_threads() -> int:
    return lib().oracle_num_threads()
