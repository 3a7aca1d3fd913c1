// capi.hip -- the extern "C" boundary declared in include/slc.h: host-side
// argument validation, workspace arithmetic and kernel launches.  Nothing
// here allocates, synchronises or reads device memory.

#include <cmath>
#include <cstdint>
#include <mutex>
#include <cstdio>
#include <cstring>

#include "slc_internal.hpp"

using namespace slc;

namespace {

thread_local char g_last_error[256] = "";

slc_status_t fail(const char *msg) {
    std::snprintf(g_last_error, sizeof g_last_error, "%s", msg);
    return SLC_ERR_INVALID_ARG;
}

slc_status_t hip_status(hipError_t e) {
    if (e == hipSuccess) return SLC_OK;
    std::snprintf(g_last_error, sizeof g_last_error, "HIP: %s", hipGetErrorString(e));
    return SLC_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

slc_status_t check_pool(const slc_pool_t &p, const char *name) {
    const char *why = nullptr;
    if (!p.base || !p.block_table) why = "base and block_table are required";
    else if (!aligned(p.base, 16)) why = "base must be 16-byte aligned";
    else if (p.table_stride < 1 || p.n_blocks < 0 || p.n_blocks > (int64_t(1) << 24))
        why = "table_stride must be >= 1 and n_blocks in [0, 2^24]";
    if (!why) return SLC_OK;
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", name, why);
    return SLC_ERR_INVALID_ARG;
}

bool heads_ok(int h, int max_h) { return h >= 16 && h <= max_h && h % 16 == 0; }

}  // namespace

extern "C" {

const char *slc_status_string(slc_status_t s) {
    switch (s) {
    case SLC_OK: return "ok";
    case SLC_ERR_INVALID_ARG: return "invalid argument";
    case SLC_ERR_WORKSPACE: return "workspace too small";
    case SLC_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

const char *slc_last_error(void) { return g_last_error; }

slc_status_t slc_compress(int ratio, int n_seq, const int32_t *cu_seqlens, int max_seqlen,
                          const uint16_t *kv, const float *score, const float *gamma, float eps,
                          const float *cos_sin, int max_pos, slc_pool_t cmp_pool,
                          float *prequant, void *stream) {
    if (ratio != 4 && ratio != 128) return fail("compress: ratio must be 4 or 128");
    if (n_seq < 1 || n_seq > 65535) return fail("compress: n_seq must be in [1, 65535]");
    if (max_seqlen < 0 || max_pos < 0) return fail("compress: max_seqlen and max_pos must be >= 0");
    if (!cu_seqlens || !kv || !score || !gamma || !cos_sin)
        return fail("compress: cu_seqlens, kv, score, gamma and cos_sin are required");
    if (!aligned(kv, 16) || !aligned(score, 16) || !aligned(gamma, 16) ||
        (prequant && !aligned(prequant, 16)))
        return fail("compress: kv, score, gamma and prequant must be 16-byte aligned");
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail("compress: eps must be finite and >= 0");
    slc_status_t st = check_pool(cmp_pool, "compress: cmp_pool");
    if (st != SLC_OK) return st;
    if (max_seqlen == 0) return SLC_OK;
    CompressArgs a{ratio, max_seqlen, cu_seqlens, kv, score, gamma, eps, cos_sin, max_pos,
                   cmp_pool, prequant};
    return hip_status(launch_compress(a, n_seq, static_cast<hipStream_t>(stream)));
}

static slc_status_t check_index_common(int n_q, const int32_t *q_seq, const int32_t *q_pos,
                                       int ratio, const int32_t *n_slots, int max_slots) {
    if (n_q < 0) return fail("index: n_q must be >= 0");
    if (ratio != 4 && ratio != 128) return fail("index: ratio must be 4 or 128");
    if (max_slots < 1 || max_slots > SLC_MAX_SLOTS)
        return fail("index: max_slots must be in [1, SLC_MAX_SLOTS]");
    if (n_q > 0 && (!q_seq || !q_pos || !n_slots))
        return fail("index: q_seq, q_pos and n_slots are required");
    return SLC_OK;
}

slc_status_t slc_index_scores(int n_q, int h_idx, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const int32_t *q_seq, const int32_t *q_pos,
                              int ratio, slc_pool_t key_pool, const int32_t *n_slots,
                              int max_slots, float *scores, void *stream) {
    const bool key_fp4 = (ratio & SLC_KEY_MXFP4) != 0;
    ratio &= ~SLC_KEY_MXFP4;
    slc_status_t st = check_index_common(n_q, q_seq, q_pos, ratio, n_slots, max_slots);
    if (st != SLC_OK) return st;
    if (!heads_ok(h_idx, SLC_MAX_INDEX_HEADS))
        return fail("index_scores: h_idx must be a multiple of 16 in [16, 64]");
    if (n_q == 0) return SLC_OK;
    if (!q_fp8 || !q_scale || !w || !scores)
        return fail("index_scores: q_fp8, q_scale, w and scores are required");
    if (!aligned(q_fp8, 16) || !aligned(q_scale, 16) || !aligned(w, 16))
        return fail("index_scores: q_fp8, q_scale and w must be 16-byte aligned");
    st = check_pool(key_pool, "index_scores: key_pool");
    if (st != SLC_OK) return st;
    IndexArgs a{n_q, h_idx, q_fp8, q_scale, w, q_seq, q_pos, ratio, key_pool, n_slots, max_slots,
                scores, key_fp4 ? 1 : 0};
    return hip_status(launch_index_scores(a, static_cast<hipStream_t>(stream)));
}

slc_status_t slc_topk_select(int n_q, int k, const float *scores, int max_slots,
                             const int32_t *q_seq, const int32_t *q_pos, int ratio,
                             const int32_t *n_slots, int32_t *topk_idx, int32_t *topk_len,
                             void *stream) {
    slc_status_t st = check_index_common(n_q, q_seq, q_pos, ratio, n_slots, max_slots);
    if (st != SLC_OK) return st;
    if (k < 1 || k > SLC_MAX_TOPK) return fail("topk_select: k must be in [1, SLC_MAX_TOPK]");
    if (n_q == 0) return SLC_OK;
    if (!scores || !topk_idx || !topk_len)
        return fail("topk_select: scores, topk_idx and topk_len are required");
    TopkArgs a{n_q, k, scores, max_slots, q_seq, q_pos, ratio, n_slots, topk_idx, topk_len};
    return hip_status(launch_topk(a, static_cast<hipStream_t>(stream)));
}

slc_status_t slc_topk_select_warm(int n_q, int k, const float *scores, int max_slots,
                                  const int32_t *q_seq, const int32_t *q_pos, int ratio,
                                  const int32_t *n_slots, int32_t *topk_idx, int32_t *topk_len,
                                  const uint16_t *q, int n_heads, int window, slc_pool_t swa_pool,
                                  void *stream) {
    const bool swa_fp8 = (ratio & SLC_SWA_FP8) != 0;
    ratio &= ~SLC_SWA_FP8;
    slc_status_t st = check_index_common(n_q, q_seq, q_pos, ratio, n_slots, max_slots);
    if (st != SLC_OK) return st;
    if (k < 1 || k > SLC_MAX_TOPK) return fail("topk_select_warm: k must be in [1, SLC_MAX_TOPK]");
    if (!heads_ok(n_heads, SLC_MAX_HEADS))
        return fail("topk_select_warm: n_heads must be a multiple of 16 in [16, 128]");
    if (window < 0 || window > SLC_MAX_WINDOW)
        return fail("topk_select_warm: window must be in [0, SLC_MAX_WINDOW]");
    if (n_q == 0) return SLC_OK;
    if (!scores || !topk_idx || !topk_len)
        return fail("topk_select_warm: scores, topk_idx and topk_len are required");
    if (!q || !aligned(q, 16)) return fail("topk_select_warm: q is required, 16-byte aligned");
    if (window > 0) {
        st = check_pool(swa_pool, "topk_select_warm: swa_pool");
        if (st != SLC_OK) return st;
    }
    TopkArgs a{n_q, k, scores, max_slots, q_seq, q_pos, ratio, n_slots, topk_idx, topk_len};
    a.warm_q = q;
    a.warm_heads = n_heads;
    a.warm_window = window;
    a.warm_swa = swa_pool;
    a.warm_swa_fp8 = swa_fp8 ? 1 : 0;
    return hip_status(launch_topk(a, static_cast<hipStream_t>(stream)));
}

static slc_status_t compress_stream(bool one_per_seq, int ratio, int n_tok, const int32_t *tok_seq,
                                    const int32_t *tok_pos, const uint16_t *kv, const float *score,
                                    const float *ape, slc_pool_t state_pool, int state_block,
                                    const float *gamma, float eps, const float *cos_sin, int max_pos,
                                    slc_pool_t cmp_pool, float *prequant, void *stream) {
    if (ratio != 4 && ratio != 128) return fail("compress_stream: ratio must be 4 or 128");
    if (n_tok < 0) return fail("compress_stream: n_tok must be >= 0");
    if (state_block < 1 || state_block > 1024)
        return fail("compress_stream: state_block must be in [1, 1024]");
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail("compress_stream: eps must be finite and >= 0");
    if (max_pos < 1) return fail("compress_stream: max_pos must be >= 1");
    if (n_tok == 0) return SLC_OK;
    if (!tok_seq || !tok_pos || !kv || !score || !ape || !gamma || !cos_sin)
        return fail("compress_stream: tok_seq, tok_pos, kv, score, ape, gamma and cos_sin are required");
    if (!aligned(kv, 16) || !aligned(score, 16) || !aligned(gamma, 16) ||
        (prequant && !aligned(prequant, 16)))
        return fail("compress_stream: kv, score, gamma and prequant must be 16-byte aligned");
    slc_status_t st = check_pool(state_pool, "compress_stream: state_pool");
    if (st != SLC_OK) return st;
    if (!aligned(state_pool.base, 16)) return fail("compress_stream: state_pool must be 16-byte aligned");
    st = check_pool(cmp_pool, "compress_stream: cmp_pool");
    if (st != SLC_OK) return st;
    StreamArgs a{ratio, n_tok, tok_seq, tok_pos, kv, score, ape, state_pool, state_block,
                 gamma, eps, cos_sin, max_pos, cmp_pool, prequant, kD};
    return hip_status(launch_compress_stream(a, one_per_seq, static_cast<hipStream_t>(stream)));
}

slc_status_t slc_compress_stream(int ratio, int n_tok, const int32_t *tok_seq,
                                 const int32_t *tok_pos, const uint16_t *kv, const float *score,
                                 const float *ape, slc_pool_t state_pool, int state_block,
                                 const float *gamma, float eps, const float *cos_sin, int max_pos,
                                 slc_pool_t cmp_pool, float *prequant, void *stream) {
    return compress_stream(false, ratio, n_tok, tok_seq, tok_pos, kv, score, ape, state_pool,
                           state_block, gamma, eps, cos_sin, max_pos, cmp_pool, prequant, stream);
}

slc_status_t slc_compress_stream_step(int ratio, int n_tok, const int32_t *tok_seq,
                                      const int32_t *tok_pos, const uint16_t *kv,
                                      const float *score, const float *ape,
                                      slc_pool_t state_pool, int state_block, const float *gamma,
                                      float eps, const float *cos_sin, int max_pos,
                                      slc_pool_t cmp_pool, float *prequant, void *stream) {
    return compress_stream(true, ratio, n_tok, tok_seq, tok_pos, kv, score, ape, state_pool,
                           state_block, gamma, eps, cos_sin, max_pos, cmp_pool, prequant, stream);
}

static slc_status_t index_keys_stream(bool one_per_seq, int n_tok, const int32_t *tok_seq,
                                      const int32_t *tok_pos, const uint16_t *kv,
                                      const float *score, const float *ape,
                                      slc_pool_t state_pool, int state_block,
                                      const float *gamma, float eps, const float *cos_sin,
                                      int max_pos, int key_flags, slc_pool_t key_pool,
                                      float *prequant, void *stream) {
    if (n_tok < 0) return fail("compress_index_keys_stream: n_tok must be >= 0");
    if (key_flags != 0 && key_flags != SLC_KEY_MXFP4)
        return fail("compress_index_keys_stream: key_flags must be 0 or SLC_KEY_MXFP4");
    if (state_block < 1 || state_block > 1024)
        return fail("compress_index_keys_stream: state_block must be in [1, 1024]");
    if (!(eps >= 0.f) || !std::isfinite(eps))
        return fail("compress_index_keys_stream: eps must be finite and >= 0");
    if (max_pos < 1) return fail("compress_index_keys_stream: max_pos must be >= 1");
    if (n_tok == 0) return SLC_OK;
    if (!tok_seq || !tok_pos || !kv || !score || !ape || !gamma || !cos_sin)
        return fail("compress_index_keys_stream: tok_seq, tok_pos, kv, score, ape, gamma and "
                    "cos_sin are required");
    if (!aligned(kv, 16) || !aligned(score, 16) || !aligned(gamma, 16) ||
        (prequant && !aligned(prequant, 16)))
        return fail("compress_index_keys_stream: kv, score, gamma and prequant must be 16-byte aligned");
    slc_status_t st = check_pool(state_pool, "compress_index_keys_stream: state_pool");
    if (st != SLC_OK) return st;
    if (!aligned(state_pool.base, 16))
        return fail("compress_index_keys_stream: state_pool must be 16-byte aligned");
    st = check_pool(key_pool, "compress_index_keys_stream: key_pool");
    if (st != SLC_OK) return st;
    StreamArgs a{4, n_tok, tok_seq, tok_pos, kv, score, ape, state_pool, state_block,
                 gamma, eps, cos_sin, max_pos, key_pool, prequant, kDI,
                 key_flags == SLC_KEY_MXFP4 ? 1 : 0};
    return hip_status(launch_compress_stream(a, one_per_seq, static_cast<hipStream_t>(stream)));
}

slc_status_t slc_compress_index_keys_stream(int n_tok, const int32_t *tok_seq,
                                            const int32_t *tok_pos, const uint16_t *kv,
                                            const float *score, const float *ape,
                                            slc_pool_t state_pool, int state_block,
                                            const float *gamma, float eps, const float *cos_sin,
                                            int max_pos, int key_flags, slc_pool_t key_pool,
                                            float *prequant, void *stream) {
    return index_keys_stream(false, n_tok, tok_seq, tok_pos, kv, score, ape, state_pool,
                             state_block, gamma, eps, cos_sin, max_pos, key_flags, key_pool,
                             prequant, stream);
}

slc_status_t slc_compress_index_keys_stream_step(int n_tok, const int32_t *tok_seq,
                                                 const int32_t *tok_pos, const uint16_t *kv,
                                                 const float *score, const float *ape,
                                                 slc_pool_t state_pool, int state_block,
                                                 const float *gamma, float eps,
                                                 const float *cos_sin, int max_pos, int key_flags,
                                                 slc_pool_t key_pool, float *prequant,
                                                 void *stream) {
    return index_keys_stream(true, n_tok, tok_seq, tok_pos, kv, score, ape, state_pool,
                             state_block, gamma, eps, cos_sin, max_pos, key_flags, key_pool,
                             prequant, stream);
}

slc_status_t slc_decode_step_writers(const slc_step_writers_t *w, void *stream) {
    if (!w) return fail("decode_step_writers: w is required");
    const int n = w->n_tok;
    if (n < 0) return fail("decode_step_writers: n_tok must be >= 0");
    if (n == 0) return SLC_OK;
    if (!w->tok_seq || !w->tok_pos || !w->cos_sin || w->max_pos < 1)
        return fail("decode_step_writers: tok_seq, tok_pos and cos_sin (max_pos >= 1) are required");
    slc_status_t st;
    SwaInsertArgs swa{};
    if (w->swa_kv) {
        if (!aligned(w->swa_kv, 16)) return fail("decode_step_writers: swa_kv must be 16-byte aligned");
        if ((st = check_pool(w->swa_pool, "decode_step_writers: swa_pool")) != SLC_OK) return st;
        swa = SwaInsertArgs{n, w->swa_kv, w->tok_seq, w->tok_pos, w->cos_sin, w->max_pos,
                            w->swa_pool, nullptr};
    }
    auto check_stream = [&](const uint16_t *kv, const float *score, const float *ape,
                            const float *gamma, float eps, slc_pool_t state, int block,
                            slc_pool_t dst, const char *what) -> slc_status_t {
        if (!score || !ape || !gamma)
            return fail("decode_step_writers: score, ape and gamma of each compressor are required");
        if (!aligned(kv, 16) || !aligned(score, 16) || !aligned(gamma, 16) || !aligned(state.base, 16))
            return fail("decode_step_writers: kv, score, gamma and state pools must be 16-byte aligned");
        if (block < 1 || block > 1024) return fail("decode_step_writers: state_block must be in [1, 1024]");
        if (!(eps >= 0.f) || !std::isfinite(eps)) return fail("decode_step_writers: eps must be finite and >= 0");
        slc_status_t r = check_pool(state, "decode_step_writers: state_pool");
        if (r != SLC_OK) return r;
        return check_pool(dst, what);
    };
    StreamArgs lat{}, keys{};
    if (w->kv) {
        if (w->ratio != 4 && w->ratio != 128) return fail("decode_step_writers: ratio must be 4 or 128");
        if ((st = check_stream(w->kv, w->score, w->ape, w->gamma, w->eps, w->state_pool,
                               w->state_block, w->cmp_pool, "decode_step_writers: cmp_pool")) != SLC_OK)
            return st;
        lat = StreamArgs{w->ratio, n, w->tok_seq, w->tok_pos, w->kv, w->score, w->ape,
                         w->state_pool, w->state_block, w->gamma, w->eps, w->cos_sin, w->max_pos,
                         w->cmp_pool, nullptr, kD};
    }
    if (w->key_kv) {
        if (w->key_flags != 0 && w->key_flags != SLC_KEY_MXFP4)
            return fail("decode_step_writers: key_flags must be 0 or SLC_KEY_MXFP4");
        if ((st = check_stream(w->key_kv, w->key_score, w->key_ape, w->key_gamma, w->key_eps,
                               w->key_state_pool, w->key_state_block, w->key_pool,
                               "decode_step_writers: key_pool")) != SLC_OK)
            return st;
        keys = StreamArgs{4, n, w->tok_seq, w->tok_pos, w->key_kv, w->key_score, w->key_ape,
                          w->key_state_pool, w->key_state_block, w->key_gamma, w->key_eps,
                          w->cos_sin, w->max_pos, w->key_pool, nullptr, kDI,
                          w->key_flags == SLC_KEY_MXFP4 ? 1 : 0};
    }
    return hip_status(launch_step_writers(w->kv ? &lat : nullptr, w->key_kv ? &keys : nullptr,
                                          w->swa_kv ? &swa : nullptr,
                                          static_cast<hipStream_t>(stream)));
}

slc_status_t slc_swa_insert(int n_tok, const uint16_t *kv, const int32_t *tok_seq,
                            const int32_t *tok_pos, const float *cos_sin, int max_pos,
                            slc_pool_t swa_pool, float *prequant_debug, void *stream) {
    if (n_tok < 0) return fail("swa_insert: n_tok must be >= 0");
    if (max_pos < 1) return fail("swa_insert: max_pos must be >= 1");
    if (n_tok == 0) return SLC_OK;
    if (!kv || !tok_seq || !tok_pos || !cos_sin)
        return fail("swa_insert: kv, tok_seq, tok_pos and cos_sin are required");
    if (!aligned(kv, 16) || (prequant_debug && !aligned(prequant_debug, 16)))
        return fail("swa_insert: kv and prequant_debug must be 16-byte aligned");
    slc_status_t st = check_pool(swa_pool, "swa_insert: swa_pool");
    if (st != SLC_OK) return st;
    SwaInsertArgs a{n_tok, kv, tok_seq, tok_pos, cos_sin, max_pos, swa_pool, prequant_debug};
    return hip_status(launch_swa_insert(a, static_cast<hipStream_t>(stream)));
}

slc_status_t slc_indexcache_skips(int n_layers, const int32_t *compress_ratios, int freq,
                                  const char *pattern, int32_t *skip) {
    if (n_layers < 0) return fail("indexcache_skips: n_layers must be >= 0");
    if (n_layers == 0) return SLC_OK;
    if (!compress_ratios || !skip) return fail("indexcache_skips: compress_ratios and skip are required");
    size_t plen = 0;
    if (pattern) {
        plen = std::strlen(pattern);
        if (plen > 0 && pattern[0] != 'F')
            return fail("indexcache_skips: a pattern must begin with 'F'");
        for (size_t i = 0; i < plen; i++)
            if (pattern[i] != 'F' && pattern[i] != 'S')
                return fail("indexcache_skips: a pattern holds only 'F' and 'S'");
    }
    // a ratio-4 layer's place among the ratio-4 layers decides; others never reuse
    int64_t seq = 0;
    for (int l = 0; l < n_layers; l++) {
        if (compress_ratios[l] != 4) {
            skip[l] = 0;
            continue;
        }
        bool reuse;
        if (plen > 0) reuse = seq < static_cast<int64_t>(plen) && pattern[seq] == 'S';
        else reuse = freq > 1 && seq % freq != 0;
        skip[l] = reuse ? 1 : 0;
        seq++;
    }
    return SLC_OK;
}

size_t slc_index_topk_workspace_size(int n_q, int max_slots) {
    if (n_q <= 0 || max_slots <= 0) return 0;
    return (static_cast<size_t>(n_q) * static_cast<size_t>(max_slots) * sizeof(float) + 255) &
           ~static_cast<size_t>(255);
}

slc_status_t slc_index_topk(int n_q, int h_idx, int k, const uint8_t *q_fp8,
                            const float *q_scale, const float *w, const int32_t *q_seq,
                            const int32_t *q_pos, int ratio, slc_pool_t key_pool,
                            const int32_t *n_slots, int max_slots, int32_t *topk_idx,
                            int32_t *topk_len, void *workspace, size_t ws_bytes, void *stream) {
    const int r = ratio & ~SLC_KEY_MXFP4;        // the key format flag goes to the scores only
    slc_status_t st = check_index_common(n_q, q_seq, q_pos, r, n_slots, max_slots);
    if (st != SLC_OK) return st;
    if (k < 1 || k > SLC_MAX_TOPK) return fail("index_topk: k must be in [1, SLC_MAX_TOPK]");
    if (!heads_ok(h_idx, SLC_MAX_INDEX_HEADS))
        return fail("index_topk: h_idx must be a multiple of 16 in [16, 64]");
    if (n_q == 0) return SLC_OK;
    size_t need = slc_index_topk_workspace_size(n_q, max_slots);
    if (!workspace || ws_bytes < need || !aligned(workspace, 256)) {
        std::snprintf(g_last_error, sizeof g_last_error,
                      "index_topk: workspace needs %zu bytes, 256-byte aligned", need);
        return SLC_ERR_WORKSPACE;
    }
    float *scores = static_cast<float *>(workspace);
    st = slc_index_scores(n_q, h_idx, q_fp8, q_scale, w, q_seq, q_pos, ratio, key_pool, n_slots,
                          max_slots, scores, stream);
    if (st != SLC_OK) return st;
    return slc_topk_select(n_q, k, scores, max_slots, q_seq, q_pos, r, n_slots, topk_idx,
                           topk_len, stream);
}

static size_t attn_ws(int n_q, int n_heads, int window, int k, bool decode) {
    if (n_q <= 0 || n_heads <= 0) return 0;
    int splits, cps, groups;
    attention_plan(n_q, n_heads, window, k, decode, &splits, &cps, &groups);
    if (splits <= 1) return 0;
    size_t per = static_cast<size_t>(n_q) * splits * n_heads;
    // bf16 normalised outputs, then (max, sum) pairs on a 16-byte boundary
    size_t bytes = ((per * kDN * sizeof(uint16_t) + 15) & ~static_cast<size_t>(15)) +
                   per * 2 * sizeof(float) + 256;
    return (bytes + 255) & ~static_cast<size_t>(255);
}

size_t slc_sparse_mla_decode_workspace_size(int n_q, int n_heads, int window, int k) {
    return attn_ws(n_q, n_heads, window, k, true);
}

size_t slc_sparse_mla_prefill_workspace_size(int n_q, int n_heads, int window, int k) {
    return attn_ws(n_q, n_heads, window, k, false);
}

size_t slc_workspace_size(slc_op_t op, const slc_shape_t *shape) {
    if (!shape) return SIZE_MAX;
    switch (op) {
    case SLC_OP_INDEX_TOPK: return slc_index_topk_workspace_size(shape->n_q, shape->max_slots);
    case SLC_OP_SPARSE_MLA_DECODE:
        return attn_ws(shape->n_q, shape->n_heads, shape->window, shape->k, true);
    case SLC_OP_SPARSE_MLA_PREFILL:
        return attn_ws(shape->n_q, shape->n_heads, shape->window, shape->k, false);
    }
    return SIZE_MAX;
}

// The attention calls' argument checks (everything but the workspace).
static slc_status_t mla_args_check(int layer_type, int n_q, int n_heads, const uint16_t *q,
                                   const int32_t *q_seq, const int32_t *q_pos, int window,
                                   slc_pool_t swa_pool, slc_pool_t cmp_pool,
                                   const int32_t *cmp_idx, int k, const int32_t *n_slots,
                                   float sm_scale, uint16_t *out) {
    layer_type &= ~SLC_SWA_FP8;
    if (layer_type != SLC_LAYER_SWAONLY && layer_type != SLC_LAYER_C4A &&
        layer_type != SLC_LAYER_C128A)
        return fail("sparse_mla: layer_type must be SWAONLY (1), C4A (4) or C128A (128), "
                    "optionally with SLC_SWA_FP8");
    if (n_q < 0) return fail("sparse_mla: n_q must be >= 0");
    if (!heads_ok(n_heads, SLC_MAX_HEADS))
        return fail("sparse_mla: n_heads must be a multiple of 16 in [16, 128]");
    if (window < 0 || window > SLC_MAX_WINDOW)
        return fail("sparse_mla: window must be in [0, SLC_MAX_WINDOW]");
    if (k < 0 || k > SLC_MAX_TOPK) return fail("sparse_mla: k must be in [0, SLC_MAX_TOPK]");
    if (layer_type == SLC_LAYER_SWAONLY && k != 0)
        return fail("sparse_mla: a SWAONLY layer takes no compressed list (k must be 0)");
    if (!std::isfinite(sm_scale)) return fail("sparse_mla: sm_scale must be finite");
    if (n_q == 0) return SLC_OK;
    if (!q || !q_seq || !q_pos || !out) return fail("sparse_mla: q, q_seq, q_pos and out are required");
    if (!aligned(q, 16) || !aligned(out, 16))
        return fail("sparse_mla: q and out must be 16-byte aligned");
    slc_status_t st;
    if (window > 0) {
        st = check_pool(swa_pool, "sparse_mla: swa_pool");
        if (st != SLC_OK) return st;
    }
    if (layer_type != SLC_LAYER_SWAONLY) {
        st = check_pool(cmp_pool, "sparse_mla: cmp_pool");
        if (st != SLC_OK) return st;
        if (k > 0 && (!cmp_idx || !n_slots))
            return fail("sparse_mla: cmp_idx and n_slots are required for C4A / C128A");
    }
    return SLC_OK;
}

static slc_status_t sparse_mla(bool decode, int layer_type, int n_q, int n_heads,
                               const uint16_t *q, const int32_t *q_seq, const int32_t *q_pos,
                               int window, slc_pool_t swa_pool, slc_pool_t cmp_pool,
                               const int32_t *cmp_idx, int k, const int32_t *n_slots,
                               float sm_scale, uint16_t *out, float *lse, void *workspace,
                               size_t ws_bytes, void *stream) {
    slc_status_t st = mla_args_check(layer_type, n_q, n_heads, q, q_seq, q_pos, window, swa_pool,
                                     cmp_pool, cmp_idx, k, n_slots, sm_scale, out);
    if (st != SLC_OK || n_q == 0) return st;
    const bool swa_fp8 = (layer_type & SLC_SWA_FP8) != 0;
    layer_type &= ~SLC_SWA_FP8;
    int kk = layer_type == SLC_LAYER_SWAONLY ? 0 : k;
    int splits, cps, groups;
    attention_plan(n_q, n_heads, window, kk, decode, &splits, &cps, &groups);
    size_t need = attn_ws(n_q, n_heads, window, kk, decode);
    if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256))) {
        std::snprintf(g_last_error, sizeof g_last_error,
                      "sparse_mla: workspace needs %zu bytes, 256-byte aligned", need);
        return SLC_ERR_WORKSPACE;
    }
    AttnArgs a{};
    a.layer_type = layer_type;
    a.n_q = n_q;
    a.n_heads = n_heads;
    a.q = q;
    a.q_seq = q_seq;
    a.q_pos = q_pos;
    a.window = window;
    a.swa_fp8 = swa_fp8 ? 1 : 0;
    a.swa = swa_pool;
    a.cmp = cmp_pool;
    a.cmp_idx = cmp_idx;
    a.k = kk;
    a.n_slots = n_slots;
    a.sm_scale_log2 = sm_scale * kLog2e;
    a.out = out;
    a.lse = lse;
    a.n_splits = splits;
    a.rows_per_split = cps;
    a.head_groups = groups;
    if (splits > 1) {
        size_t per = static_cast<size_t>(n_q) * splits * n_heads;
        a.part_o = static_cast<uint16_t *>(workspace);
        a.part_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                              ((per * kDN * sizeof(uint16_t) + 15) & ~static_cast<size_t>(15)));
    }
    return hip_status(launch_attention(a, decode, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ------------------------------------------------------- no-allocation decode
// The decode's split partials in a library-owned device array instead of a
// caller workspace.  In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns for the
// current device may reach a kernel or a copy.  Each GPU holds its own copy
// until the process ends.
namespace {

constexpr size_t kScratchBytes = size_t(12) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address, resolved once per device.
slc_status_t scratch_of_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return fail("sparse_mla_decode_noalloc: device id out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!ptr) return fail("sparse_mla_decode_noalloc: no device address for the scratch array");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SLC_OK;
}

}  // namespace

extern "C" {

size_t slc_sparse_mla_decode_noalloc_max_bytes(void) { return kScratchBytes; }

slc_status_t slc_sparse_mla_decode_noalloc(int layer_type, int n_q, int n_heads,
                                           const uint16_t *q, const int32_t *q_seq,
                                           const int32_t *q_pos, int window, slc_pool_t swa_pool,
                                           slc_pool_t cmp_pool, const int32_t *cmp_idx, int k,
                                           const int32_t *n_slots, float sm_scale, uint16_t *out,
                                           float *lse, void *stream) {
    // the argument and size checks are host arithmetic and come before any
    // device call
    slc_status_t st0 = mla_args_check(layer_type, n_q, n_heads, q, q_seq, q_pos, window, swa_pool,
                                      cmp_pool, cmp_idx, k, n_slots, sm_scale, out);
    if (st0 != SLC_OK || n_q == 0) return st0;
    const int kk = (layer_type & ~SLC_SWA_FP8) == SLC_LAYER_SWAONLY ? 0 : k;
    const size_t need = n_q > 0 && n_heads > 0 && kk >= 0 && window >= 0
                            ? attn_ws(n_q, n_heads, window, kk, true) : 0;
    if (need > kScratchBytes) {
        std::snprintf(g_last_error, sizeof g_last_error,
                      "sparse_mla_decode_noalloc: these shapes need %zu bytes of split partials, "
                      "above the %zu-byte static scratch; use slc_sparse_mla_decode with a workspace",
                      need, kScratchBytes);
        return SLC_ERR_WORKSPACE;
    }
    void *ws = nullptr;
    if (need > 0) {
        slc_status_t st = scratch_of_current_device(&ws);
        if (st != SLC_OK) return st;
    }
    return sparse_mla(true, layer_type, n_q, n_heads, q, q_seq, q_pos, window, swa_pool, cmp_pool,
                      cmp_idx, k, n_slots, sm_scale, out, lse, ws, need, stream);
}

slc_status_t slc_sparse_mla_decode_topk(int layer_type, int n_q, int n_heads, const uint16_t *q,
                                        const int32_t *q_seq, const int32_t *q_pos, int window,
                                        slc_pool_t swa_pool, slc_pool_t cmp_pool, int k,
                                        const float *scores, int max_slots,
                                        const int32_t *n_slots, int32_t *topk_idx,
                                        int32_t *topk_len, float sm_scale, uint16_t *out,
                                        float *lse, void *workspace, size_t ws_bytes,
                                        void *stream) {
    if ((layer_type & ~SLC_SWA_FP8) != SLC_LAYER_C4A)
        return fail("sparse_mla_decode_topk: layer_type must be SLC_LAYER_C4A (optionally | SLC_SWA_FP8)");
    if (k < 1 || k > SLC_MAX_TOPK) return fail("sparse_mla_decode_topk: k must be in [1, SLC_MAX_TOPK]");
    slc_status_t st = check_index_common(n_q, q_seq, q_pos, SLC_LAYER_C4A, n_slots, max_slots);
    if (st != SLC_OK) return st;
    st = mla_args_check(layer_type, n_q, n_heads, q, q_seq, q_pos, window, swa_pool, cmp_pool,
                        topk_idx, k, n_slots, sm_scale, out);
    if (st != SLC_OK || n_q == 0) return st;
    if (!scores || !topk_len) return fail("sparse_mla_decode_topk: scores and topk_len are required");
    const size_t need = attn_ws(n_q, n_heads, window, k, true);
    if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256))) {
        std::snprintf(g_last_error, sizeof g_last_error,
                      "sparse_mla_decode_topk: workspace needs %zu bytes, 256-byte aligned", need);
        return SLC_ERR_WORKSPACE;
    }
    AttnArgs a{};
    a.layer_type = SLC_LAYER_C4A;
    a.n_q = n_q;
    a.n_heads = n_heads;
    a.q = q;
    a.q_seq = q_seq;
    a.q_pos = q_pos;
    a.window = window;
    a.swa_fp8 = (layer_type & SLC_SWA_FP8) ? 1 : 0;
    a.swa = swa_pool;
    a.cmp = cmp_pool;
    a.cmp_idx = topk_idx;
    a.k = k;
    a.n_slots = n_slots;
    a.sm_scale_log2 = sm_scale * kLog2e;
    a.out = out;
    a.lse = lse;
    int splits, cps, groups;
    attention_plan(n_q, n_heads, window, k, true, &splits, &cps, &groups);
    a.n_splits = splits;
    a.rows_per_split = cps;
    a.head_groups = groups;
    if (splits > 1) {
        size_t per = static_cast<size_t>(n_q) * splits * n_heads;
        a.part_o = static_cast<uint16_t *>(workspace);
        a.part_ml = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                              ((per * kDN * sizeof(uint16_t) + 15) & ~static_cast<size_t>(15)));
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (decode_can_select(a, scores, max_slots)) {
        a.sel_scores = scores;
        a.sel_max_slots = max_slots;
        a.sel_ratio = SLC_LAYER_C4A;
        a.sel_idx = topk_idx;
        a.sel_len = topk_len;
        return hip_status(launch_attention(a, true, s));
    }
    TopkArgs ta{n_q, k, scores, max_slots, q_seq, q_pos, SLC_LAYER_C4A, n_slots, topk_idx, topk_len};
    hipError_t e = launch_topk(ta, s);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(launch_attention(a, true, s));
}

slc_status_t slc_sparse_mla_decode(int layer_type, int n_q, int n_heads, const uint16_t *q,
                                   const int32_t *q_seq, const int32_t *q_pos, int window,
                                   slc_pool_t swa_pool, slc_pool_t cmp_pool,
                                   const int32_t *cmp_idx, int k, const int32_t *n_slots,
                                   float sm_scale, uint16_t *out, float *lse, void *workspace,
                                   size_t ws_bytes, void *stream) {
    return sparse_mla(true, layer_type, n_q, n_heads, q, q_seq, q_pos, window, swa_pool, cmp_pool,
                      cmp_idx, k, n_slots, sm_scale, out, lse, workspace, ws_bytes, stream);
}

slc_status_t slc_sparse_mla_prefill(int layer_type, int n_q, int n_heads, const uint16_t *q,
                                    const int32_t *q_seq, const int32_t *q_pos, int window,
                                    slc_pool_t swa_pool, slc_pool_t cmp_pool,
                                    const int32_t *cmp_idx, int k, const int32_t *n_slots,
                                    float sm_scale, uint16_t *out, float *lse, void *workspace,
                                    size_t ws_bytes, void *stream) {
    return sparse_mla(false, layer_type, n_q, n_heads, q, q_seq, q_pos, window, swa_pool,
                      cmp_pool, cmp_idx, k, n_slots, sm_scale, out, lse, workspace, ws_bytes,
                      stream);
}

}  // extern "C"
