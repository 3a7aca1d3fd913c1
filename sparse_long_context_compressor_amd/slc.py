"""Thin Python binding of libslc.so (argument marshalling only).

Every function here has the name of the C entry point without its ``slc_``
prefix and forwards torch tensors' device pointers plus torch's current HIP
stream.  All computation happens in the library's HIP kernels; there is no
fallback: if libslc.so is missing, importing functions raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

from . import pools as P

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libslc.so")

LAYER_SWAONLY, LAYER_C4A, LAYER_C128A = 1, 4, 128
SWA_FP8 = 0x100     # OR'ed into a layer type (or the warm select's ratio): fp8 SWA pool
KEY_MXFP4 = 0x200   # OR'ed into the ratio of index_scores / index_topk: MXFP4 keys
SLC_OK, SLC_ERR_INVALID_ARG, SLC_ERR_WORKSPACE, SLC_ERR_HIP = 0, 1, 2, 3

EXPORTED = [
    "slc_status_string", "slc_last_error", "slc_compress", "slc_index_scores",
    "slc_topk_select", "slc_topk_select_warm", "slc_index_topk_workspace_size", "slc_index_topk",
    "slc_indexcache_skips", "slc_swa_insert", "slc_compress_stream",
    "slc_compress_index_keys_stream", "slc_compress_stream_step",
    "slc_compress_index_keys_stream_step", "slc_decode_step_writers",
    "slc_sparse_mla_decode_workspace_size", "slc_sparse_mla_decode",
    "slc_sparse_mla_prefill_workspace_size", "slc_sparse_mla_prefill", "slc_workspace_size",
    "slc_sparse_mla_decode_noalloc", "slc_sparse_mla_decode_noalloc_max_bytes",
    "slc_sparse_mla_decode_topk",
]

OP_INDEX_TOPK, OP_SPARSE_MLA_DECODE, OP_SPARSE_MLA_PREFILL = 1, 2, 3


class Pool(C.Structure):
    _fields_ = [("base", C.c_void_p), ("block_table", C.c_void_p),
                ("table_stride", C.c_int32), ("n_blocks", C.c_int64)]


class StepWriters(C.Structure):
    _fields_ = [("n_tok", C.c_int), ("tok_seq", C.c_void_p), ("tok_pos", C.c_void_p),
                ("cos_sin", C.c_void_p), ("max_pos", C.c_int),
                ("swa_kv", C.c_void_p), ("swa_pool", Pool),
                ("ratio", C.c_int), ("kv", C.c_void_p), ("score", C.c_void_p),
                ("ape", C.c_void_p), ("gamma", C.c_void_p), ("eps", C.c_float),
                ("state_pool", Pool), ("state_block", C.c_int), ("cmp_pool", Pool),
                ("key_kv", C.c_void_p), ("key_score", C.c_void_p), ("key_ape", C.c_void_p),
                ("key_gamma", C.c_void_p), ("key_eps", C.c_float), ("key_state_pool", Pool),
                ("key_state_block", C.c_int), ("key_flags", C.c_int), ("key_pool", Pool)]


class Shape(C.Structure):
    _fields_ = [("n_q", C.c_int), ("n_heads", C.c_int), ("window", C.c_int), ("k", C.c_int),
                ("max_slots", C.c_int)]


class SlcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"slc status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libslc.so (build it with sparse_long_context_compressor_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python sparse_long_context_compressor_amd/build.py`")
        L = C.CDLL(LIB_PATH)
        i32, sz, vp, f32 = C.c_int, C.c_size_t, C.c_void_p, C.c_float
        pool = Pool
        L.slc_status_string.restype = C.c_char_p
        L.slc_status_string.argtypes = [i32]
        L.slc_last_error.restype = C.c_char_p
        L.slc_last_error.argtypes = []
        L.slc_compress.restype = i32
        L.slc_compress.argtypes = [i32, i32, vp, i32, vp, vp, vp, f32, vp, i32, pool, vp, vp]
        L.slc_index_scores.restype = i32
        L.slc_index_scores.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32, pool, vp, i32, vp, vp]
        L.slc_topk_select.restype = i32
        L.slc_topk_select.argtypes = [i32, i32, vp, i32, vp, vp, i32, vp, vp, vp, vp]
        L.slc_topk_select_warm.restype = i32
        L.slc_topk_select_warm.argtypes = [i32, i32, vp, i32, vp, vp, i32, vp, vp, vp, vp, i32, i32,
                                           pool, vp]
        for name in ("slc_compress_stream", "slc_compress_stream_step"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [i32, i32, vp, vp, vp, vp, vp, pool, i32, vp, f32, vp, i32, pool, vp, vp]
        for name in ("slc_compress_index_keys_stream", "slc_compress_index_keys_stream_step"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [i32, vp, vp, vp, vp, vp, pool, i32, vp, f32, vp, i32, i32, pool, vp, vp]
        L.slc_decode_step_writers.restype = i32
        L.slc_decode_step_writers.argtypes = [C.POINTER(StepWriters), vp]
        L.slc_swa_insert.restype = i32
        L.slc_swa_insert.argtypes = [i32, vp, vp, vp, vp, i32, pool, vp, vp]
        L.slc_indexcache_skips.restype = i32
        L.slc_indexcache_skips.argtypes = [i32, vp, i32, C.c_char_p, vp]
        L.slc_index_topk_workspace_size.restype = sz
        L.slc_index_topk_workspace_size.argtypes = [i32, i32]
        L.slc_index_topk.restype = i32
        L.slc_index_topk.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, i32, pool, vp, i32, vp,
                                     vp, vp, sz, vp]
        for name in ("slc_sparse_mla_decode", "slc_sparse_mla_prefill"):
            f = getattr(L, name)
            f.restype = i32
            f.argtypes = [i32, i32, i32, vp, vp, vp, i32, pool, pool, vp, i32, vp, f32, vp, vp,
                          vp, sz, vp]
            g = getattr(L, name + "_workspace_size")
            g.restype = sz
            g.argtypes = [i32, i32, i32, i32]
        L.slc_sparse_mla_decode_noalloc.restype = i32
        L.slc_sparse_mla_decode_noalloc.argtypes = [i32, i32, i32, vp, vp, vp, i32, pool, pool, vp,
                                                    i32, vp, f32, vp, vp, vp]
        L.slc_sparse_mla_decode_noalloc_max_bytes.restype = sz
        L.slc_sparse_mla_decode_noalloc_max_bytes.argtypes = []
        L.slc_workspace_size.restype = sz
        L.slc_workspace_size.argtypes = [i32, C.POINTER(Shape)]
        L.slc_sparse_mla_decode_topk.restype = i32
        L.slc_sparse_mla_decode_topk.argtypes = [i32, i32, i32, vp, vp, vp, i32, pool, pool, i32,
                                                 vp, i32, vp, vp, vp, f32, vp, vp, vp, sz, vp]
        _lib = L
    return _lib


def _check(status: int):
    if status != SLC_OK:
        L = lib()
        raise SlcError(status, L.slc_last_error().decode() or L.slc_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, dev):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name}: expected device {dev}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def pool(base: Optional[torch.Tensor], table: Optional[torch.Tensor]) -> Pool:
    """slc_pool_t over a pool tensor [n_blocks, ...] and its block table [n_seq, stride]."""
    if base is None:
        return Pool(None, None, 0, 0)
    if table.dtype != torch.int32 or not table.is_contiguous():
        raise TypeError("block table must be contiguous int32")
    return Pool(base.data_ptr(), table.data_ptr(), int(table.shape[1]), int(base.shape[0]))


def _bits16(t: torch.Tensor) -> torch.Tensor:
    return t if t.dtype == torch.int16 else t.view(torch.int16)


# ----------------------------------------------------------------- compress
def compress(ratio: int, cu_seqlens: torch.Tensor, max_seqlen: int, kv: torch.Tensor,
             score: torch.Tensor, gamma: torch.Tensor, eps: float, cos_sin: torch.Tensor,
             cmp_pool: torch.Tensor, cmp_table: torch.Tensor,
             prequant: Optional[torch.Tensor] = None) -> None:
    dev = kv.device
    _need(kv, "kv", torch.bfloat16, dev)
    _need(score, "score", torch.float32, dev)
    _need(gamma, "gamma", torch.float32, dev)
    _need(cos_sin, "cos_sin", torch.float32, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _need(cmp_pool, "cmp_pool", torch.uint8, dev)
    if prequant is not None:
        _need(prequant, "prequant", torch.float32, dev)
    _check(lib().slc_compress(int(ratio), int(cu_seqlens.numel() - 1), _ptr(cu_seqlens),
                              int(max_seqlen), _ptr(kv), _ptr(score), _ptr(gamma), float(eps),
                              _ptr(cos_sin), int(cos_sin.shape[0]), pool(cmp_pool, cmp_table),
                              _ptr(prequant), _stream()))


def compress_stream(ratio: int, tok_seq: torch.Tensor, tok_pos: torch.Tensor, kv: torch.Tensor,
                    score: torch.Tensor, ape: torch.Tensor, state_pool: torch.Tensor,
                    state_table: torch.Tensor, state_block: int, gamma: torch.Tensor, eps: float,
                    cos_sin: torch.Tensor, cmp_pool: torch.Tensor, cmp_table: torch.Tensor,
                    prequant: Optional[torch.Tensor] = None, one_per_seq: bool = False) -> None:
    """One step of the streaming compressor: state rows of the given tokens,
    then the slots they complete (state_pool fp32 [n_blocks, state_block,
    2*coff*576]).  one_per_seq: at most one token per sequence, one launch."""
    dev = kv.device
    _need(kv, "kv", torch.bfloat16, dev)
    _need(score, "score", torch.float32, dev)
    _need(ape, "ape", torch.float32, dev)
    _need(state_pool, "state_pool", torch.float32, dev)
    _need(gamma, "gamma", torch.float32, dev)
    _need(cos_sin, "cos_sin", torch.float32, dev)
    _need(tok_seq, "tok_seq", torch.int32, dev)
    _need(tok_pos, "tok_pos", torch.int32, dev)
    _need(cmp_pool, "cmp_pool", torch.uint8, dev)
    if prequant is not None:
        _need(prequant, "prequant", torch.float32, dev)
    f = lib().slc_compress_stream_step if one_per_seq else lib().slc_compress_stream
    _check(f(int(ratio), int(kv.shape[0]), _ptr(tok_seq), _ptr(tok_pos),
                                     _ptr(kv), _ptr(score), _ptr(ape),
                                     pool(state_pool, state_table), int(state_block), _ptr(gamma),
                                     float(eps), _ptr(cos_sin), int(cos_sin.shape[0]),
                                     pool(cmp_pool, cmp_table), _ptr(prequant), _stream()))


def compress_index_keys_stream(tok_seq, tok_pos, kv, score, ape, state_pool, state_table,
                               state_block: int, gamma, eps: float, cos_sin, key_pool,
                               key_table, prequant=None, mxfp4: bool = False,
                               one_per_seq: bool = False) -> None:
    """One step of the indexer's 128-dim key compressor (ratio 4) into the
    index key pool (a KEY4 pool of MXFP4 keys with mxfp4=True); state_pool
    fp32 [n_blocks, state_block, 512]."""
    dev = kv.device
    _need(kv, "kv", torch.bfloat16, dev)
    _need(score, "score", torch.float32, dev)
    _need(ape, "ape", torch.float32, dev)
    _need(state_pool, "state_pool", torch.float32, dev)
    _need(gamma, "gamma", torch.float32, dev)
    _need(cos_sin, "cos_sin", torch.float32, dev)
    _need(tok_seq, "tok_seq", torch.int32, dev)
    _need(tok_pos, "tok_pos", torch.int32, dev)
    _need(key_pool, "key_pool", torch.uint8, dev)
    if prequant is not None:
        _need(prequant, "prequant", torch.float32, dev)
    f = (lib().slc_compress_index_keys_stream_step if one_per_seq
         else lib().slc_compress_index_keys_stream)
    _check(f(
        int(kv.shape[0]), _ptr(tok_seq), _ptr(tok_pos), _ptr(kv), _ptr(score), _ptr(ape),
        pool(state_pool, state_table), int(state_block), _ptr(gamma), float(eps), _ptr(cos_sin),
        int(cos_sin.shape[0]), KEY_MXFP4 if mxfp4 else 0, pool(key_pool, key_table),
        _ptr(prequant), _stream()))


def decode_step_writers(tok_seq, tok_pos, cos_sin, swa=None, latent=None, keys=None) -> None:
    """A decode step's writers in one launch (at most one token per sequence).
    swa = dict(kv, pool, table); latent = dict(ratio, kv, score, ape, gamma,
    eps, state, state_table, state_block, pool, table); keys = the same
    without ratio, plus mxfp4 (bool).  Omitted parts are skipped."""
    w = StepWriters()
    w.n_tok = int(tok_seq.numel())
    w.tok_seq, w.tok_pos, w.cos_sin = _ptr(tok_seq), _ptr(tok_pos), _ptr(cos_sin)
    w.max_pos = int(cos_sin.shape[0])
    if swa is not None:
        _need(swa["kv"], "swa kv", torch.bfloat16, swa["kv"].device)
        w.swa_kv, w.swa_pool = _ptr(swa["kv"]), pool(swa["pool"], swa["table"])
    if latent is not None:
        w.ratio = int(latent["ratio"])
        w.kv, w.score, w.ape = _ptr(latent["kv"]), _ptr(latent["score"]), _ptr(latent["ape"])
        w.gamma, w.eps = _ptr(latent["gamma"]), float(latent["eps"])
        w.state_pool = pool(latent["state"], latent["state_table"])
        w.state_block = int(latent["state_block"])
        w.cmp_pool = pool(latent["pool"], latent["table"])
    if keys is not None:
        w.key_kv, w.key_score, w.key_ape = _ptr(keys["kv"]), _ptr(keys["score"]), _ptr(keys["ape"])
        w.key_gamma, w.key_eps = _ptr(keys["gamma"]), float(keys["eps"])
        w.key_state_pool = pool(keys["state"], keys["state_table"])
        w.key_state_block = int(keys["state_block"])
        w.key_flags = KEY_MXFP4 if keys.get("mxfp4") else 0
        w.key_pool = pool(keys["pool"], keys["table"])
    _check(lib().slc_decode_step_writers(C.byref(w), _stream()))


def swa_insert(kv: torch.Tensor, tok_seq: torch.Tensor, tok_pos: torch.Tensor,
               cos_sin: torch.Tensor, swa_pool: torch.Tensor, swa_table: torch.Tensor,
               prequant: Optional[torch.Tensor] = None) -> None:
    """RoPE + fp8 row format + paged write of new tokens into an fp8 SWA pool
    (CMP layout); attend to it with layer_type | SWA_FP8."""
    dev = kv.device
    _need(kv, "kv", torch.bfloat16, dev)
    _need(tok_seq, "tok_seq", torch.int32, dev)
    _need(tok_pos, "tok_pos", torch.int32, dev)
    _need(cos_sin, "cos_sin", torch.float32, dev)
    _need(swa_pool, "swa_pool", torch.uint8, dev)
    if prequant is not None:
        _need(prequant, "prequant", torch.float32, dev)
    _check(lib().slc_swa_insert(int(kv.shape[0]), _ptr(kv), _ptr(tok_seq), _ptr(tok_pos),
                                _ptr(cos_sin), int(cos_sin.shape[0]), pool(swa_pool, swa_table),
                                _ptr(prequant), _stream()))


# ------------------------------------------------------------------ indexer
def index_scores(q_fp8, q_scale, w, q_seq, q_pos, ratio, key_pool, key_table, n_slots,
                 max_slots, scores) -> None:
    n_q, h_idx = int(q_fp8.shape[0]), int(q_fp8.shape[1])
    _check(lib().slc_index_scores(n_q, h_idx, _ptr(q_fp8), _ptr(q_scale), _ptr(w), _ptr(q_seq),
                                  _ptr(q_pos), int(ratio), pool(key_pool, key_table),
                                  _ptr(n_slots), int(max_slots), _ptr(scores), _stream()))


def topk_select(k, scores, max_slots, q_seq, q_pos, ratio, n_slots, topk_idx, topk_len) -> None:
    n_q = int(q_seq.numel())
    _check(lib().slc_topk_select(n_q, int(k), _ptr(scores), int(max_slots), _ptr(q_seq),
                                 _ptr(q_pos), int(ratio), _ptr(n_slots), _ptr(topk_idx),
                                 _ptr(topk_len), _stream()))


def topk_select_warm(k, scores, max_slots, q_seq, q_pos, ratio, n_slots, topk_idx, topk_len,
                     q, window, swa_pool, swa_table) -> None:
    """topk_select plus the L2 warm-up of the decode's queries and window rows."""
    n_q = int(q_seq.shape[0])
    _check(lib().slc_topk_select_warm(n_q, int(k), _ptr(scores), int(max_slots), _ptr(q_seq),
                                      _ptr(q_pos), int(ratio), _ptr(n_slots), _ptr(topk_idx),
                                      _ptr(topk_len), _ptr(q), int(q.shape[1]), int(window),
                                      pool(swa_pool, swa_table), _stream()))


def indexcache_skips(compress_ratios, freq: int, pattern: str = "") -> list:
    """Per layer 1 = reuse an earlier layer's top-k, 0 = compute (host only)."""
    import numpy as np
    r = np.ascontiguousarray(np.asarray(compress_ratios, dtype=np.int32))
    out = np.zeros(r.shape[0], np.int32)
    _check(lib().slc_indexcache_skips(int(r.shape[0]), r.ctypes.data, int(freq),
                                      pattern.encode() if pattern else None, out.ctypes.data))
    return out.tolist()


def workspace_size(op: int, n_q: int = 0, n_heads: int = 0, window: int = 0, k: int = 0,
                   max_slots: int = 0) -> int:
    """slc_workspace_size: bytes of workspace the call `op` needs for these
    shapes (OP_INDEX_TOPK, OP_SPARSE_MLA_DECODE, OP_SPARSE_MLA_PREFILL)."""
    sh = Shape(int(n_q), int(n_heads), int(window), int(k), int(max_slots))
    return int(lib().slc_workspace_size(int(op), C.byref(sh)))


def index_topk_workspace_size(n_q: int, max_slots: int) -> int:
    return int(lib().slc_index_topk_workspace_size(int(n_q), int(max_slots)))


def index_topk(k, q_fp8, q_scale, w, q_seq, q_pos, ratio, key_pool, key_table, n_slots,
               max_slots, topk_idx, topk_len, workspace: Optional[torch.Tensor] = None) -> None:
    n_q, h_idx = int(q_fp8.shape[0]), int(q_fp8.shape[1])
    need = index_topk_workspace_size(n_q, max_slots)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q_fp8.device)
    _check(lib().slc_index_topk(n_q, h_idx, int(k), _ptr(q_fp8), _ptr(q_scale), _ptr(w),
                                _ptr(q_seq), _ptr(q_pos), int(ratio), pool(key_pool, key_table),
                                _ptr(n_slots), int(max_slots), _ptr(topk_idx), _ptr(topk_len),
                                _ptr(workspace), int(workspace.numel()), _stream()))


# ---------------------------------------------------------------- attention
def sparse_mla_workspace_size(decode: bool, n_q: int, n_heads: int, window: int, k: int) -> int:
    f = (lib().slc_sparse_mla_decode_workspace_size if decode
         else lib().slc_sparse_mla_prefill_workspace_size)
    return int(f(int(n_q), int(n_heads), int(window), int(k)))


def _sparse_mla(decode, layer_type, q, q_seq, q_pos, window, swa_pool, swa_table, cmp_pool,
                cmp_table, cmp_idx, n_slots, sm_scale, out, lse, workspace):
    n_q, H = int(q.shape[0]), int(q.shape[1])
    k = 0 if cmp_idx is None else int(cmp_idx.shape[1])
    need = sparse_mla_workspace_size(decode, n_q, H, window, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    f = lib().slc_sparse_mla_decode if decode else lib().slc_sparse_mla_prefill
    _check(f(int(layer_type), n_q, H, _ptr(q), _ptr(q_seq), _ptr(q_pos), int(window),
             pool(swa_pool, swa_table), pool(cmp_pool, cmp_table), _ptr(cmp_idx), k,
             _ptr(n_slots), float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
             0 if workspace is None else int(workspace.numel()), _stream()))


def sparse_mla_decode(layer_type, q, q_seq, q_pos, window, swa_pool, swa_table, cmp_pool=None,
                      cmp_table=None, cmp_idx=None, n_slots=None, sm_scale=1.0, out=None,
                      lse=None, workspace=None):
    _sparse_mla(True, layer_type, q, q_seq, q_pos, window, swa_pool, swa_table, cmp_pool,
                cmp_table, cmp_idx, n_slots, sm_scale, out, lse, workspace)


def sparse_mla_prefill(layer_type, q, q_seq, q_pos, window, swa_pool, swa_table, cmp_pool=None,
                       cmp_table=None, cmp_idx=None, n_slots=None, sm_scale=1.0, out=None,
                       lse=None, workspace=None):
    _sparse_mla(False, layer_type, q, q_seq, q_pos, window, swa_pool, swa_table, cmp_pool,
                cmp_table, cmp_idx, n_slots, sm_scale, out, lse, workspace)


def sparse_mla_decode_topk(layer_type, q, q_seq, q_pos, window, swa_pool, swa_table, cmp_pool,
                           cmp_table, k, scores, max_slots, n_slots, topk_idx, topk_len,
                           sm_scale=1.0, out=None, lse=None, workspace=None):
    """slc_sparse_mla_decode_topk: the C4A top-k select of scores and the decode
    over its list in one call (the list also written to topk_idx / topk_len)."""
    n_q, H = int(q.shape[0]), int(q.shape[1])
    need = sparse_mla_workspace_size(True, n_q, H, window, int(k))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().slc_sparse_mla_decode_topk(
        int(layer_type), n_q, H, _ptr(q), _ptr(q_seq), _ptr(q_pos), int(window),
        pool(swa_pool, swa_table), pool(cmp_pool, cmp_table), int(k), _ptr(scores),
        int(max_slots), _ptr(n_slots), _ptr(topk_idx), _ptr(topk_len), float(sm_scale), _ptr(out),
        _ptr(lse), _ptr(workspace), 0 if workspace is None else int(workspace.numel()), _stream()))


def sparse_mla_decode_noalloc(layer_type, q, q_seq, q_pos, window, swa_pool, swa_table,
                              cmp_pool=None, cmp_table=None, cmp_idx=None, n_slots=None,
                              sm_scale=1.0, out=None, lse=None):
    """slc_sparse_mla_decode_noalloc: the decode with its split partials in the
    library's static device array (no workspace, no allocation)."""
    n_q, H = int(q.shape[0]), int(q.shape[1])
    k = 0 if cmp_idx is None else int(cmp_idx.shape[1])
    _check(lib().slc_sparse_mla_decode_noalloc(
        int(layer_type), n_q, H, _ptr(q), _ptr(q_seq), _ptr(q_pos), int(window),
        pool(swa_pool, swa_table), pool(cmp_pool, cmp_table), _ptr(cmp_idx), k, _ptr(n_slots),
        float(sm_scale), _ptr(out), _ptr(lse), _stream()))


def sparse_mla_decode_noalloc_max_bytes() -> int:
    return int(lib().slc_sparse_mla_decode_noalloc_max_bytes())
