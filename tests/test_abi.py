"""CPU checks of the boundary: the library exports every symbol include/slc.h
declares, argument errors are returned before any launch, and the binding
fails loudly without the library.  No compute call is made here."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "slc.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def S():
    from sparse_long_context_compressor_amd import slc
    if not os.path.exists(slc.LIB_PATH):
        from sparse_long_context_compressor_amd import build
        build.build()
    try:
        slc.lib()
    except OSError as e:  # the HIP runtime itself is not loadable here
        pytest.skip(f"cannot load libslc.so: {e}")
    return slc


def test_exports_every_declared_symbol(S):
    names = declared_symbols()
    assert len(names) >= 11
    L = S.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(S.EXPORTED) == set(names)


def test_status_strings(S):
    L = S.lib()
    assert L.slc_status_string(0) == b"ok"
    assert L.slc_status_string(2) == b"workspace too small"


def _null_pool(S):
    return S.Pool(None, None, 0, 0)


def test_invalid_arguments_are_rejected_before_launch(S):
    L = S.lib()
    P = _null_pool(S)
    fake = C.c_void_p(256)   # never dereferenced: validation fails first
    # ratio 3 is not a compress ratio
    assert L.slc_compress(3, 1, fake, 8, fake, fake, fake, 1e-6, fake, 8, P, None, None) == 1
    assert b"ratio" in L.slc_last_error()
    # a ratio-4 compress without a destination pool
    assert L.slc_compress(4, 1, fake, 8, fake, fake, fake, 1e-6, fake, 8, P, None, None) == 1
    assert b"cmp_pool" in L.slc_last_error()
    # indexer heads must be a multiple of 16 up to 64
    assert L.slc_index_scores(1, 20, fake, fake, fake, fake, fake, 4, P, fake, 16, fake, None) == 1
    assert L.slc_index_scores(1, 80, fake, fake, fake, fake, fake, 4, P, fake, 16, fake, None) == 1
    # k above the cap
    assert L.slc_topk_select(1, 5000, fake, 16, fake, fake, 4, fake, fake, fake, None) == 1
    # layer type 2 does not exist; SWAONLY takes no compressed list
    args = [1, 64, fake, fake, fake, 128, P, P, None, 0, None, 0.1, fake, None, None, 0, None]
    assert L.slc_sparse_mla_decode(2, *args) == 1
    a2 = list(args)
    a2[9] = 8
    assert L.slc_sparse_mla_decode(1, *a2) == 1
    # C4A without its compressed pool
    a3 = list(args)
    a3[9] = 8
    a3[5] = 0
    assert L.slc_sparse_mla_decode(4, *a3) == 1
    assert b"cmp_pool" in L.slc_last_error()
    # heads not a multiple of 16
    a4 = list(args)
    a4[1] = 40
    assert L.slc_sparse_mla_decode(1, *a4) == 1
    # misaligned q
    a5 = list(args)
    a5[2] = C.c_void_p(258)
    a5[5] = 0
    assert L.slc_sparse_mla_decode(1, *a5) == 1
    # a decode that needs a workspace but gets none
    pool = S.Pool(C.c_void_p(256), C.c_void_p(256), 4, 4)
    a6 = [32, 64, fake, fake, fake, 128, pool, pool, fake, 512, fake, 0.1, fake, None, None, 0, None]
    assert L.slc_sparse_mla_decode(4, *a6) == 2
    assert L.slc_sparse_mla_decode_workspace_size(32, 64, 128, 512) > 0
    assert L.slc_sparse_mla_prefill_workspace_size(2048, 64, 128, 2048) == 0
    # nothing to do is not an error
    assert L.slc_topk_select(0, 8, None, 16, None, None, 4, None, None, None, None) == 0


def test_decode_topk_validates_on_the_host(S):
    """slc_sparse_mla_decode_topk: argument and workspace errors come back
    before any launch (no device here)."""
    L = S.lib()
    fake = C.c_void_p(256)
    pool = S.Pool(C.c_void_p(256), C.c_void_p(256), 4, 4)

    def call(layer, k, ws=None, ws_bytes=0, scores=fake, max_slots=16384, topk_len=fake):
        return L.slc_sparse_mla_decode_topk(layer, 32, 64, fake, fake, fake, 128, pool, pool, k,
                                            scores, max_slots, fake, fake, topk_len, 0.1, fake,
                                            None, ws, ws_bytes, None)
    assert call(128, 512) == 1 and b"C4A" in L.slc_last_error()      # C128A takes a given list
    assert call(1, 512) == 1                                           # SWAONLY has no list
    assert call(4, 0) == 1 and call(4, 5000) == 1                      # k outside 1..SLC_MAX_TOPK
    assert call(4, 512, max_slots=0) == 1                              # no slots
    assert call(4, 512, scores=None) == 1 and b"scores" in L.slc_last_error()
    assert call(4, 512, topk_len=None) == 1
    assert call(4, 512) == 2                                           # the decode's workspace is missing
    assert L.slc_sparse_mla_decode_topk(4, 0, 64, None, None, None, 128, pool, pool, 512, None,
                                        16384, None, None, None, 0.1, None, None, None, 0,
                                        None) == 0                     # nothing to do is not an error


def test_workspace_size_dispatches_to_the_per_op_sizers(S):
    """slc_workspace_size (host arithmetic) equals the matching per-op sizer on
    every workload shape and on edge shapes, and flags misuse with SIZE_MAX."""
    L = S.lib()
    size_max = C.c_size_t(-1).value
    shapes = [(32, 64, 128, 512, 16384), (64, 64, 128, 0, 1), (32, 64, 128, 512, 1024),
              (2048, 64, 128, 2048, 32768), (1, 16, 128, 256, 1024), (1, 128, 1024, 4096, 5000),
              (0, 64, 128, 512, 16384), (3, 48, 64, 77, 1000), (5, 16, 0, 0, 1)]
    for n_q, h, w, k, ms in shapes:
        sh = S.Shape(n_q, h, w, k, ms)
        assert L.slc_workspace_size(S.OP_INDEX_TOPK, C.byref(sh)) == \
            L.slc_index_topk_workspace_size(n_q, ms)
        assert L.slc_workspace_size(S.OP_SPARSE_MLA_DECODE, C.byref(sh)) == \
            L.slc_sparse_mla_decode_workspace_size(n_q, h, w, k)
        assert L.slc_workspace_size(S.OP_SPARSE_MLA_PREFILL, C.byref(sh)) == \
            L.slc_sparse_mla_prefill_workspace_size(n_q, h, w, k)
        assert S.workspace_size(S.OP_SPARSE_MLA_DECODE, n_q, h, w, k, ms) == \
            L.slc_sparse_mla_decode_workspace_size(n_q, h, w, k)
    # the index scores of 32 queries over 16384 slots, 256-byte rounded
    sh = S.Shape(32, 64, 128, 512, 16384)
    assert L.slc_workspace_size(S.OP_INDEX_TOPK, C.byref(sh)) == 32 * 16384 * 4
    assert L.slc_workspace_size(S.OP_SPARSE_MLA_DECODE, C.byref(sh)) > 0
    assert L.slc_workspace_size(S.OP_SPARSE_MLA_PREFILL, C.byref(sh)) == 0
    # an unknown op or no shape: SIZE_MAX, which no allocation satisfies
    assert L.slc_workspace_size(9, C.byref(sh)) == size_max
    assert L.slc_workspace_size(S.OP_INDEX_TOPK, None) == size_max


def test_noalloc_decode_rejects_oversized_shapes_before_any_device_call(S):
    """The no-allocation decode checks its partials' size against its static
    array on the host (SLC_ERR_WORKSPACE), before it touches a device."""
    L = S.lib()
    assert L.slc_sparse_mla_decode_noalloc_max_bytes() == 12 << 20
    fake = C.c_void_p(256)
    pool = S.Pool(C.c_void_p(256), C.c_void_p(256), 4, 4)
    # 100 queries x 2 head blocks split in two: 13 MB of partials
    assert L.slc_sparse_mla_decode_workspace_size(100, 64, 128, 512) > (12 << 20)
    assert L.slc_sparse_mla_decode_workspace_size(32, 64, 128, 512) <= (12 << 20)
    st = L.slc_sparse_mla_decode_noalloc(4, 100, 64, fake, fake, fake, 128, pool, pool, fake,
                                         512, fake, 0.1, fake, None, None)
    assert st == 2 and b"static scratch" in L.slc_last_error()
    # argument errors come first, as for the workspace form
    assert L.slc_sparse_mla_decode_noalloc(2, 1, 64, fake, fake, fake, 128, pool, pool, None, 0,
                                           None, 0.1, fake, None, None) == 1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from sparse_long_context_compressor_amd import slc
    monkeypatch.setattr(slc, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(slc, "_lib", None)
    with pytest.raises(ImportError):
        slc.lib()


def test_package_never_imports_the_oracle():
    """The product package never imports, loads or runs anything under oracle/."""
    pat = re.compile(r"(^\s*(import|from)\s+oracle\b)|liboracle|slc_oracle|oracle_[a-z]+\(",
                     re.M)
    pkg = os.path.join(ROOT, "sparse_long_context_compressor_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat.search(text), os.path.join(dirpath, f)


def test_indexcache_skips_match_the_oracle(S, oracle):
    """The library's schedule (host arithmetic) against the oracle's, on random
    ratio layouts, frequencies and patterns, plus its argument errors."""
    import numpy as np
    rng = np.random.default_rng(3)
    for _ in range(200):
        n = int(rng.integers(0, 60))
        ratios = rng.choice([1, 4, 4, 4, 128], size=n).tolist()
        freq = int(rng.integers(0, 6))
        pattern = ""
        if rng.random() < 0.4:
            m = int(rng.integers(1, 12))
            pattern = "F" + "".join(rng.choice(["F", "S"], size=m - 1).tolist())
        assert S.indexcache_skips(ratios, freq, pattern) == oracle.indexcache_skips(ratios, freq, pattern)
    with pytest.raises(S.SlcError):
        S.indexcache_skips([4, 4], 2, "SF")
    with pytest.raises(S.SlcError):
        S.indexcache_skips([4, 4], 2, "FX")


def test_invalid_arguments_of_the_next_rows_are_rejected(S):
    """The fp8 SWA insert, the streaming compressors and the MXFP4 flag
    validate on the host, before any launch."""
    L = S.lib()
    P = _null_pool(S)
    fake = C.c_void_p(256)
    pool = S.Pool(C.c_void_p(256), C.c_void_p(256), 4, 4)
    # SWA insert: no destination pool; misaligned kv; nothing to do is fine
    assert L.slc_swa_insert(2, fake, fake, fake, fake, 16, P, None, None) == 1
    assert L.slc_swa_insert(2, C.c_void_p(258), fake, fake, fake, 16, pool, None, None) == 1
    assert L.slc_swa_insert(0, None, None, None, None, 16, P, None, None) == 0
    # streaming compressor: ratio, state block size, missing pools
    a = [1, fake, fake, fake, fake, fake, pool, 4, fake, 1e-6, fake, 16, pool, None, None]
    assert L.slc_compress_stream(3, *a) == 1 and b"ratio" in L.slc_last_error()
    b = list(a)
    b[7] = 0
    assert L.slc_compress_stream(4, *b) == 1 and b"state_block" in L.slc_last_error()
    c = list(a)
    c[6] = P
    assert L.slc_compress_stream(4, *c) == 1 and b"state_pool" in L.slc_last_error()
    d = list(a)
    d[12] = P
    assert L.slc_compress_stream(128, *d) == 1 and b"cmp_pool" in L.slc_last_error()
    e = [1, fake, fake, fake, fake, fake, pool, 4, fake, 1e-6, fake, 16, 0, P, None, None]
    assert L.slc_compress_index_keys_stream(*e) == 1 and b"key_pool" in L.slc_last_error()
    f = list(e)
    f[9] = -1.0
    assert L.slc_compress_index_keys_stream(*f) == 1 and b"eps" in L.slc_last_error()
    h = list(e)
    h[12] = 3
    assert L.slc_compress_index_keys_stream(*h) == 1 and b"key_flags" in L.slc_last_error()
    # the MXFP4 flag does not make an invalid ratio valid; the SWA flag on a
    # layer type that does not exist is rejected
    assert L.slc_index_scores(1, 16, fake, fake, fake, fake, fake, 3 | S.KEY_MXFP4, P, fake, 16,
                              fake, None) == 1
    args = [1, 64, fake, fake, fake, 128, P, P, None, 0, None, 0.1, fake, None, None, 0, None]
    assert L.slc_sparse_mla_decode(2 | S.SWA_FP8, *args) == 1


def test_decode_step_writers_validate_on_the_host(S):
    L = S.lib()
    assert L.slc_decode_step_writers(None, None) == 1
    w = S.StepWriters()
    w.n_tok = 0
    assert L.slc_decode_step_writers(C.byref(w), None) == 0            # nothing to do
    fake = 256
    w.n_tok, w.tok_seq, w.tok_pos, w.cos_sin, w.max_pos = 4, fake, fake, fake, 16
    w.kv, w.score, w.ape, w.gamma, w.ratio = fake, fake, fake, fake, 3
    assert L.slc_decode_step_writers(C.byref(w), None) == 1 and b"ratio" in L.slc_last_error()
    w.kv = None
    w.key_kv, w.key_score, w.key_ape, w.key_gamma, w.key_flags = fake, fake, fake, fake, 7
    assert L.slc_decode_step_writers(C.byref(w), None) == 1 and b"key_flags" in L.slc_last_error()
    w.key_flags = 0
    assert L.slc_decode_step_writers(C.byref(w), None) == 1 and b"state" in L.slc_last_error()
    w.key_kv = None
    w.swa_kv = 258                                                        # misaligned
    assert L.slc_decode_step_writers(C.byref(w), None) == 1 and b"swa_kv" in L.slc_last_error()
