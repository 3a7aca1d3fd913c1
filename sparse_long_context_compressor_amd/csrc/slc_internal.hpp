// slc_internal.hpp -- kernel argument blocks and launch entry points shared
// between the C-ABI layer (capi.hip) and the kernel translation units.
#pragma once

#include "slc_device.hpp"

namespace slc {

struct CompressArgs {
    int ratio;
    int max_seqlen;
    const int32_t *cu_seqlens;
    const uint16_t *kv;
    const float *score;
    const float *gamma;
    float eps;
    const float *cos_sin;
    int max_pos;
    slc_pool_t pool;
    float *prequant;
};

// SWA KV insert: token t (sequence tok_seq[t], position tok_pos[t]) of kv
// [n_tok][576] bf16 -> row tok_pos[t] of its sequence in a pool of the
// compressed-row layout; prequant (nullable) [n_tok][576] fp32.
struct SwaInsertArgs {
    int n_tok;
    const uint16_t *kv;
    const int32_t *tok_seq;
    const int32_t *tok_pos;
    const float *cos_sin;
    int max_pos;
    slc_pool_t pool;
    float *prequant;
};

// Streaming compressor: token t (sequence tok_seq[t], position tok_pos[t])
// brings coff kv / score blocks; its state row (fp32: coff kv blocks, then
// coff score blocks with the APE bias added) lives in a paged state pool of
// state_block rows per block; a token that completes a slot emits it.
struct StreamArgs {
    int ratio;
    int n_tok;
    const int32_t *tok_seq;
    const int32_t *tok_pos;
    const uint16_t *kv;         // [n_tok][coff*576] bf16
    const float *score;         // [n_tok][coff*576]
    const float *ape;           // [ratio][coff*576]
    slc_pool_t state;
    int state_block;
    const float *gamma;
    float eps;
    const float *cos_sin;
    int max_pos;
    slc_pool_t pool;            // compressed pool (CMP layout; KEY layout for dim 128)
    float *prequant;            // nullable [n_tok][dim], rows of emitting tokens
    int dim;                    // 576 (latent rows) or 128 (index keys, ratio 4)
    int key_fp4;                // index keys: MXFP4 into a KEY4 pool instead of fp8
};

struct IndexArgs {
    int n_q;
    int h_idx;
    const uint8_t *q;
    const float *q_scale;
    const float *w;
    const int32_t *q_seq;
    const int32_t *q_pos;
    int ratio;
    slc_pool_t keys;
    const int32_t *n_slots;
    int max_slots;
    float *scores;
    int key_fp4;            // keys: MXFP4 (KEY4 layout) instead of fp8 + fp32 scale
};

struct TopkArgs {
    int n_q;
    int k;
    const float *scores;
    int max_slots;
    const int32_t *q_seq;
    const int32_t *q_pos;
    int ratio;
    const int32_t *n_slots;
    int32_t *idx;
    int32_t *len;
    // optional L2 warm-up for the attention that follows (warm_q null: none):
    // query t's heads warm_q[t][warm_heads][576] and the latent rows of its
    // window (positions p - warm_window + 1 .. p) in warm_swa
    const uint16_t *warm_q;
    int warm_heads;
    int warm_window;
    slc_pool_t warm_swa;
    int warm_swa_fp8;       // warm_swa holds fp8 rows in the compressed-row layout
};

struct AttnArgs {
    int layer_type;
    int n_q;
    int n_heads;
    const uint16_t *q;
    const int32_t *q_seq;
    const int32_t *q_pos;
    int window;
    int swa_fp8;            // swa holds fp8 rows in the compressed-row layout
    slc_pool_t swa;
    slc_pool_t cmp;
    const int32_t *cmp_idx;
    int k;
    const int32_t *n_slots;
    float sm_scale_log2;    // sm_scale * log2(e)
    uint16_t *out;
    float *lse;
    int n_splits;           // decode: workgroups per (query, head block) along the list
    int rows_per_split;     // prefill: list entries of its one split
    int head_groups;        // decode: 16-head groups per workgroup (1 or 2)
    int sw_per, cm_per;     // decode: window / compressed entries per split
    int sw_cap, cm_cap;     // decode: window / compressed rows per LDS pass
    uint16_t *part_o;       // bf16 [n_q][n_splits][H][512] (decode, n_splits > 1)
    float *part_ml;         // [n_q][n_splits][H][2]
    // decode that selects its own compressed list (sel_scores non-null):
    // index scores [n_q][sel_max_slots], visible counts by sel_ratio; the
    // list goes to sel_idx [n_q][k] and its length to sel_len [n_q]
    const float *sel_scores;
    int sel_max_slots;
    int sel_ratio;
    int32_t *sel_idx;
    int32_t *sel_len;
};

hipError_t launch_compress(const CompressArgs &a, int n_seq, hipStream_t stream);
hipError_t launch_swa_insert(const SwaInsertArgs &a, hipStream_t stream);
hipError_t launch_compress_stream(const StreamArgs &a, bool one_per_seq, hipStream_t stream);
hipError_t launch_step_writers(const StreamArgs *lat, const StreamArgs *keys,
                               const SwaInsertArgs *swa, hipStream_t stream);
hipError_t launch_index_scores(const IndexArgs &a, hipStream_t stream);
hipError_t launch_topk(const TopkArgs &a, hipStream_t stream);
hipError_t launch_attention(const AttnArgs &a, bool decode, hipStream_t stream);
hipError_t launch_decode(const AttnArgs &a, hipStream_t stream);   // decode.hip (no combine)
// whether launch_decode selects the list itself for these shapes (else the
// caller runs the top-k select first)
bool decode_can_select(const AttnArgs &a, const float *scores, int max_slots);
hipError_t launch_combine(const AttnArgs &a, hipStream_t stream);  // merge of the decode's splits

// split plan (host arithmetic only): decode splits each (query, head block)'s
// lists so that about one workgroup per CU runs; prefill never splits.
void attention_plan(int n_q, int n_heads, int window, int k, bool decode, int *n_splits,
                    int *rows_per_split, int *head_groups);
// 16-head groups one decode workgroup serves (2 when n_heads allows, else 1)

}  // namespace slc
