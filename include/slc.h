/*
 * slc.h -- C ABI of the MI355X (gfx950) compressed sparse attention library.
 *
 * One DeepSeek-V4-style attention layer with compressed history, in four
 * calls (plus the two stages of the indexer on their own):
 *
 *   slc_compress            softmax-gated pooling of ratio-r token windows,
 *                           RMSNorm, RoPE at the slot anchor, FP8 quantisation,
 *                           paged store.
 *   slc_index_scores        lightning-indexer scores of FP8 index queries
 *                           against the FP8 index keys of the visible slots.
 *   slc_topk_select         per-query global top-k over those scores.
 *   slc_index_topk          the two above in one call.
 *   slc_compress_stream     the same compressor step by step: per-token state
 *                           rows (two kv/score blocks, APE bias), slots
 *                           emitted as they complete.
 *   slc_compress_index_keys_stream  the indexer's 128-dim key compressor,
 *                           step by step, into the index key pool.
 *   slc_decode_step_writers the per-token writers of a decode step (SWA insert
 *                           and both streaming compressors) in one launch.
 *   slc_swa_insert          RoPE + fp8 quantisation + paged write of new tokens
 *                           into an fp8 sliding-window pool
 *   slc_sparse_mla_decode_topk  the C4A top-k select and the decode over its
 *                           list in one call.
 *   slc_sparse_mla_decode   absorbed-MQA sparse MLA attention over the sliding
 *   slc_sparse_mla_prefill  window plus the selected compressed slots.
 *
 * Sources, by page title and section:
 *   "DeepSeek-V4 attention layer types" (juejin.cn post 7667401749827403791):
 *       layer-type table (compress_ratio 1 / 4 / 128 -> swaonly / c4a /
 *       c128a), "Compressor" (window overlap, anchor (pos//r)*r), "Indexer,
 *       C4A and C128A top-k" (c4a computes a global top-k per step, c128a
 *       takes a precomputed list; FlashMLA takes SWA and compressed indices).
 *   "DeepseekV4Attention" (devpress.csdn.net, AMD): DeepseekCompressor
 *       forward and its kernel arguments, CSA compressor formula and
 *       boundary table, cache block layout, Indexer formula, forward_mqa,
 *       _forward_prefill / _forward_decode call surfaces.
 *   "From MLA to CSA + HCA" (forceinjection.github.io): Ch.2 absorbed MLA
 *       (576-wide latent, values from its first 512 dims), 5.1 CSA, 5.2 HCA,
 *       6.1 precisions, 6.3 compressed slot mapping.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers are device memory owned by the caller unless stated.  The
 *   library allocates nothing, keeps no global state and never synchronises
 *   the stream or reads device memory on the host; every call only enqueues
 *   kernels on `stream` (a hipStream_t passed as void*; NULL = null stream).
 * - Argument errors are found on the host before any launch and returned as
 *   SLC_ERR_INVALID_ARG (nothing is enqueued); a too-small workspace is
 *   SLC_ERR_WORKSPACE; a failed launch is SLC_ERR_HIP.  Nothing throws.
 * - Device-side index contents (block tables, slot and position lists) are
 *   never trusted: entries that are negative or out of range are skipped,
 *   never dereferenced.
 * - bf16 is passed as its 16-bit pattern (uint16_t), fp8 as OCP E4M3FN
 *   bytes (bias 7, max 448, no infinities) -- the fp8 format of gfx950.
 * - Paged pools: each pool is n_blocks blocks of SLC_BLOCK_ROWS rows; row j
 *   of sequence b lives in physical block block_table[b*table_stride + j/64]
 *   at row j%64.  Table entries < 0 or >= n_blocks mean "absent": reads of
 *   such rows are skipped, writes to them are dropped.
 *
 * Pool byte layouts (per block):
 *   SWA pool  bf16 [64][576]                                   73728 B
 *   CMP pool  rows: 64 x (512 e4m3 codes | 64 bf16 rope) = 640 B each,
 *             then scales: 64 x 8 fp32 (one per 64 nope dims)   43008 B
 *   KEY pool  codes: 64 x 128 e4m3, then scales: 64 x fp32        8448 B
 * (the pages store row data first and the block's scales after all its rows;
 * this library keeps that order with its own row widths).
 * A pool holds at most 2^24 blocks (physical row ids fit in int32); larger
 * n_blocks is SLC_ERR_INVALID_ARG.  base must be 16-byte aligned.
 * CMP scales are powers of two (slc_compress writes nothing else): code *
 * scale is then exact in bf16.  A pool filled by other means with other
 * positive scales is dequantised with one bf16 rounding of code * scale.
 */
#ifndef SLC_H
#define SLC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SLC_BLOCK_ROWS 64
#define SLC_D_LATENT 576        /* 512 nope + 64 rope */
#define SLC_D_NOPE 512          /* value width */
#define SLC_D_ROPE 64
#define SLC_D_INDEX 128         /* indexer head dim */
#define SLC_SWA_BLOCK_BYTES 73728
#define SLC_CMP_ROW_BYTES 640
#define SLC_CMP_SCALE_OFFSET 40960
#define SLC_CMP_BLOCK_BYTES 43008
#define SLC_KEY_SCALE_OFFSET 8192
#define SLC_KEY_BLOCK_BYTES 8448
#define SLC_KEY4_SCALE_OFFSET 4096  /* MXFP4 key block: 64 x 64 B e2m1 pairs, */
#define SLC_KEY4_BLOCK_BYTES 4352   /* then 64 x 4 E8M0 scale bytes           */

#define SLC_MAX_HEADS 128       /* query heads: a multiple of 16, <= 128 */
#define SLC_MAX_INDEX_HEADS 64  /* indexer heads: a multiple of 16, <= 64 */
#define SLC_MAX_TOPK 4096
#define SLC_MAX_WINDOW 1024
#define SLC_MAX_SLOTS 1048576   /* compressed slots per sequence */

typedef enum {
    SLC_OK = 0,
    SLC_ERR_INVALID_ARG = 1,
    SLC_ERR_WORKSPACE = 2,
    SLC_ERR_HIP = 3
} slc_status_t;

/* Layer types keyed by compress ratio ("DeepSeek-V4 attention layer types",
 * layer-type table): swaonly attends the window only; c4a adds the indexer's
 * top-k slots; c128a adds a given (precomputed) slot list. */
typedef enum {
    SLC_LAYER_SWAONLY = 1,
    SLC_LAYER_C4A = 4,
    SLC_LAYER_C128A = 128
} slc_layer_t;

/* Flag OR'ed into the layer type of slc_sparse_mla_decode / _prefill (and
 * into the ratio of slc_topk_select_warm): the SWA pool holds fp8 rows in the
 * compressed-row (CMP) layout, as slc_swa_insert writes them, instead of
 * bf16 rows ("From MLA to CSA + HCA" 5.5: the V4 SWA cache stores fp8 nope
 * dims, bf16 rope dims and one scale per 64 dims). */
#define SLC_SWA_FP8 0x100

/* Flag OR'ed into the ratio of slc_index_scores / slc_index_topk: the key
 * pool holds MXFP4 keys (the KEY4 layout: per key 128 e2m1 values, two per
 * byte with the even element in the low nibble, and one E8M0 scale byte per
 * 32 dims, 68 bytes in all) instead of fp8 keys with one fp32 scale.  "From
 * MLA to CSA + HCA" 6.1 (FP4 / MXFP4 indexer K cache); "DeepseekV4Attention"
 * (devpress), Indexer (the FP4 indexer cache).  The scores are then
 *   I[t][s] = sum_j w[t][j] * ReLU(q_scale[t][j] * sum_d q[t][j][d] * k[s][d]),
 *   k[s][d] = e2m1 * 2^(e - 127) with e the scale byte of d's 32-dim block,
 * exact in the bf16 operands for scale bytes 2..254 (0 reads as a zero
 * block; 255, NaN in E8M0, is not a valid key). */
#define SLC_KEY_MXFP4 0x200

typedef struct slc_pool {
    void *base;                  /* device: n_blocks blocks                         */
    const int32_t *block_table;  /* device: [n_seq][table_stride] physical block ids */
    int32_t table_stride;        /* entries per sequence (logical blocks)           */
    int64_t n_blocks;            /* physical blocks in base                         */
} slc_pool_t;

/* Human-readable name of a status code (static storage). */
const char *slc_status_string(slc_status_t s);

/* Last argument error of this thread, for diagnostics (static storage). */
const char *slc_last_error(void);

/*
 * slc_compress -- "DeepseekV4Attention" (devpress), DeepseekCompressor forward
 * and the CSA compressor section; "From MLA to CSA + HCA" 5.1, 5.2, 6.3.
 *
 * For each sequence b (tokens cu_seqlens[b] .. cu_seqlens[b+1]-1, length L,
 * positions 0..L-1) and each slot j < ceil(L/ratio):
 *   window T_j = [r*j - (coff-1)*r, r*j + r - 1] clipped to [0, L), coff = 2
 *            for r = 4 (overlapping 8-token gather), 1 for r = 128;
 *   pooled[d] = sum_t softmax_t(score[t][d]) * kv[t][d], per channel d;
 *   y = pooled * gamma / sqrt(mean(pooled^2) + eps) over all 576 dims;
 *   RoPE (GPT-J interleaved pairs (512+2i, 513+2i)) at position r*j with
 *            cos = cos_sin[r*j][i], sin = cos_sin[r*j][32+i];
 *   nope dims: 8 blocks of 64 -> scale = smallest 2^e with amax <= 448*2^e
 *            (1 if amax = 0), code = e4m3(y/scale) round-to-nearest-even;
 *   rope dims: bf16 round-to-nearest-even;
 *   stored at slot j of sequence b in cmp_pool.
 * A trailing partial slot (L % r != 0) is pooled over the tokens present.
 *
 *   ratio        4 or 128
 *   n_seq        sequences (>= 1)
 *   cu_seqlens   device int32 [n_seq+1], non-decreasing, cu_seqlens[0] = 0
 *   max_seqlen   host bound on every L (sizes the grid); longer sequences
 *                are truncated to max_seqlen tokens
 *   kv           device bf16 [T][576];  score  device fp32 [T][576]
 *   gamma        device fp32 [576];     eps >= 0
 *   cos_sin      device fp32 [max_pos][64]; slots whose anchor r*j >= max_pos
 *                are not written
 *   cmp_pool     destination (CMP layout)
 *   prequant     nullable device fp32 [cmp_pool.n_blocks*64][576]: the row
 *                after RMSNorm and RoPE, at the slot's physical row (debug)
 */
slc_status_t slc_compress(int ratio, int n_seq, const int32_t *cu_seqlens, int max_seqlen,
                          const uint16_t *kv, const float *score, const float *gamma, float eps,
                          const float *cos_sin, int max_pos, slc_pool_t cmp_pool,
                          float *prequant, void *stream);

/*
 * slc_compress_stream -- the compressor as it runs step by step
 * ("DeepseekV4Attention" (devpress): DeepseekCompressor forward, where
 * save_partial_states adds the APE bias and keeps kv and score in an fp32
 * state cache, then the fused compress kernel; "CSA compressor": the C_a /
 * C_b formula and the state layout; "From MLA to CSA + HCA" 5.5: a slot is
 * compressed once its ratio-th token has arrived).
 *
 * Each token t (sequence tok_seq[t], position p = tok_pos[t]) brings coff kv
 * blocks and coff gate-score blocks of 576 dims (coff = 2 for ratio 4: C_a,
 * C_b; 1 for ratio 128).  Step 1 writes its state row:
 *   state[p] = [ kv blocks as fp32 | score blocks + ape[p % ratio] in fp32 ].
 * Step 2: a token with (p + 1) % ratio == 0 emits slot j = p / ratio from
 * the state rows of its window, per channel d:
 *   ratio 4:   positions 4j-4 .. 4j-1 with block 0, 4j .. 4j+3 with block 1;
 *   ratio 128: positions 128j .. 128j+127 with block 0;
 *   pooled[d] = softmax-weighted sum of the entries' kv over their logits
 *   (absent rows and positions < 0 are skipped),
 * then RMSNorm, RoPE at r*j, quantisation and the store exactly as
 * slc_compress.  The window's earlier rows come from earlier calls or from
 * this one (step 1 completes before step 2).
 *
 *   ratio        4 or 128
 *   n_tok        tokens in this call (>= 0); no two may share (sequence, position)
 *   tok_seq, tok_pos  device int32 [n_tok]
 *   kv           device bf16 [n_tok][coff*576], 16-byte aligned
 *   score        device fp32 [n_tok][coff*576], 16-byte aligned
 *   ape          device fp32 [ratio][coff*576]
 *   state_pool   device fp32 rows of 2*coff*576 floats, state_block rows per
 *                block, one table row per sequence (the pages use blocks of 4
 *                rows for ratio 4 and 8 for ratio 128); a window of coff*ratio
 *                positions must stay mapped until its slot is emitted
 *   gamma, eps, cos_sin, max_pos, cmp_pool  as for slc_compress
 *   prequant     nullable device fp32 [n_tok][576]: for an emitting token,
 *                its slot's row after RMSNorm and RoPE (debug)
 */
slc_status_t slc_compress_stream(int ratio, int n_tok, const int32_t *tok_seq,
                                 const int32_t *tok_pos, const uint16_t *kv, const float *score,
                                 const float *ape, slc_pool_t state_pool, int state_block,
                                 const float *gamma, float eps, const float *cos_sin, int max_pos,
                                 slc_pool_t cmp_pool, float *prequant, void *stream);

/*
 * slc_compress_stream_step -- slc_compress_stream in one launch for calls
 * that bring at most one token per sequence (a decode step): each token's
 * workgroup writes its state row and, if it completes a slot, pools the
 * window from the rows saved by earlier calls plus its own row, which it
 * keeps on chip.  Arguments and results as slc_compress_stream; a call with
 * two tokens of one sequence gives unspecified slots (never an access out of
 * bounds).
 */
slc_status_t slc_compress_stream_step(int ratio, int n_tok, const int32_t *tok_seq,
                                      const int32_t *tok_pos, const uint16_t *kv,
                                      const float *score, const float *ape,
                                      slc_pool_t state_pool, int state_block, const float *gamma,
                                      float eps, const float *cos_sin, int max_pos,
                                      slc_pool_t cmp_pool, float *prequant, void *stream);

/*
 * slc_compress_index_keys_stream -- the indexer's own compressor, step by
 * step ("DeepSeek-V4 attention layer types": the indexer holds a small
 * compressor of head_dim 128 whose entries fill its K cache;
 * "DeepseekV4Attention": the compressor class's RoPE on the last 64 dims and
 * the indexer cache entry of 128 fp8 values plus one fp32 scale).
 *
 * As slc_compress_stream with ratio 4 and rows of 128 dims: kv and score
 * [n_tok][2*128] (blocks C_a, C_b), ape [4][2*128], state rows of 4*128
 * floats.  An emitting token (p = 4j + 3) pools slot j's window, then
 *   y = pooled * gamma / sqrt(mean(pooled^2) + eps) over the 128 dims,
 *   RoPE on the pairs (64+2i, 65+2i) at position 4j (cos_sin[4j][i],
 *   cos_sin[4j][32+i]),
 *   one scale for the key (smallest 2^e with amax <= 448*2^e, 1 if amax = 0)
 *   and e4m3 codes of y / scale,
 * stored at slot j of its sequence in key_pool (KEY layout), the index keys
 * slc_index_scores reads.  With key_flags = SLC_KEY_MXFP4 the key is written
 * as MXFP4 into a KEY4 pool instead: per 32-dim block the smallest 2^e with
 * amax <= 6 * 2^e (E8M0 byte e + 127) and the nearest e2m1 code of y / 2^e,
 * ties to the even code.
 *   key_flags    0 (fp8 keys) or SLC_KEY_MXFP4
 *   gamma        device fp32 [128], 16-byte aligned
 *   prequant     nullable device fp32 [n_tok][128] (debug)
 * Other arguments as for slc_compress_stream.
 */
slc_status_t slc_compress_index_keys_stream(int n_tok, const int32_t *tok_seq,
                                            const int32_t *tok_pos, const uint16_t *kv,
                                            const float *score, const float *ape,
                                            slc_pool_t state_pool, int state_block,
                                            const float *gamma, float eps, const float *cos_sin,
                                            int max_pos, int key_flags, slc_pool_t key_pool,
                                            float *prequant, void *stream);

/*
 * slc_compress_index_keys_stream_step -- slc_compress_index_keys_stream in
 * one launch, under slc_compress_stream_step's condition (at most one token
 * per sequence per call).
 */
slc_status_t slc_compress_index_keys_stream_step(int n_tok, const int32_t *tok_seq,
                                                 const int32_t *tok_pos, const uint16_t *kv,
                                                 const float *score, const float *ape,
                                                 slc_pool_t state_pool, int state_block,
                                                 const float *gamma, float eps,
                                                 const float *cos_sin, int max_pos, int key_flags,
                                                 slc_pool_t key_pool, float *prequant,
                                                 void *stream);

/*
 * slc_decode_step_writers -- a decode step's per-token writers in one launch:
 * slc_swa_insert, slc_compress_stream_step and
 * slc_compress_index_keys_stream_step for the same n_tok tokens (at most one
 * per sequence), each part skipped when its input is NULL (swa_kv, kv,
 * key_kv).  Every part computes exactly what its own call computes; the
 * three write disjoint pools.  Arguments as in those calls.
 */
typedef struct slc_step_writers {
    int n_tok;
    const int32_t *tok_seq, *tok_pos;   /* device int32 [n_tok]               */
    const float *cos_sin;               /* device fp32 [max_pos][64]          */
    int max_pos;
    /* SWA insert: fp8 SWA pool (CMP layout) */
    const uint16_t *swa_kv;             /* [n_tok][576] bf16, or NULL         */
    slc_pool_t swa_pool;
    /* latent compressor step */
    int ratio;                          /* 4 or 128                           */
    const uint16_t *kv;                 /* [n_tok][coff*576] bf16, or NULL    */
    const float *score, *ape, *gamma;
    float eps;
    slc_pool_t state_pool;
    int state_block;
    slc_pool_t cmp_pool;
    /* index-key compressor step (ratio 4) */
    const uint16_t *key_kv;             /* [n_tok][256] bf16, or NULL         */
    const float *key_score, *key_ape, *key_gamma;
    float key_eps;
    slc_pool_t key_state_pool;
    int key_state_block;
    int key_flags;                      /* 0 or SLC_KEY_MXFP4                 */
    slc_pool_t key_pool;
} slc_step_writers_t;

slc_status_t slc_decode_step_writers(const slc_step_writers_t *w, void *stream);

/*
 * slc_swa_insert -- "From MLA to CSA + HCA" 6.2 (the fused KV insert: GPT-J
 * RoPE, fp8 quantisation and the paged write in one kernel) and 5.5 (the V4
 * SWA cache row: fp8 nope, bf16 rope, one scale per 64 dims);
 * "DeepseekV4Attention" (devpress), HCA compressor workflow, stage 3 (KV:
 * RoPE + FP8 quant + SWA cache write).
 *
 * For each token t (sequence tok_seq[t], position p = tok_pos[t]):
 *   y = kv[t] (576 dims, not yet rotated);
 *   RoPE (GPT-J interleaved pairs (512+2i, 513+2i)) at position p with
 *            cos = cos_sin[p][i], sin = cos_sin[p][32+i];
 *   nope dims: 8 blocks of 64 -> the same scale rule and e4m3 codes as
 *            slc_compress; rope dims: bf16 round-to-nearest-even;
 *   stored at row p of sequence tok_seq[t] in swa_pool.
 * Attend to such a pool with layer_type | SLC_SWA_FP8.
 *
 *   n_tok        tokens (>= 0)
 *   kv           device bf16 [n_tok][576], 16-byte aligned
 *   tok_seq, tok_pos  device int32 [n_tok]; tok_seq indexes swa_pool's table
 *   cos_sin      device fp32 [max_pos][64]; tokens with p outside
 *                [0, max_pos) are not written, nor are rows whose block is
 *                absent from the table
 *   swa_pool     destination, CMP layout (SLC_CMP_BLOCK_BYTES per block)
 *   prequant_debug  nullable device fp32 [n_tok][576], 16-byte aligned: the
 *                row after RoPE, before quantisation
 * Tokens must not share a (sequence, position): their rows would race.
 */
slc_status_t slc_swa_insert(int n_tok, const uint16_t *kv, const int32_t *tok_seq,
                            const int32_t *tok_pos, const float *cos_sin, int max_pos,
                            slc_pool_t swa_pool, float *prequant_debug, void *stream);

/*
 * slc_index_scores -- "DeepseekV4Attention" (devpress), Indexer section:
 *   I[t][s] = sum_j w[t][j] * ReLU(q_scale[t][j] * k_scale[s] * (q[t][j] . k[s]))
 * over the fp8 index query heads j < h_idx, for the slots s visible to query
 * t: s < n_vis(t) = min(n_slots[q_seq[t]], (q_pos[t]+1) / ratio)
 * ("From MLA to CSA + HCA" 5.1: position i sees slot j iff i >= r*j + r - 1).
 * fp8 products accumulate in fp32.  q_scale and the key scales must be
 * positive: the kernel applies them outside the ReLU
 * (ReLU(a*b*x) = a*b*ReLU(x) for a, b > 0).
 *
 *   n_q          queries;  h_idx  indexer heads (multiple of 16, <= 64)
 *   q_fp8        device e4m3 [n_q][h_idx][128], 16-byte aligned
 *   q_scale, w   device fp32 [n_q][h_idx], 16-byte aligned
 *   q_seq, q_pos device int32 [n_q] (sequence and position of each query)
 *   ratio        4 (the indexer exists for c4a layers), OR'ed with
 *                SLC_KEY_MXFP4 for MXFP4 keys in the KEY4 layout
 *   key_pool     KEY layout (KEY4 with SLC_KEY_MXFP4), one table row per sequence
 *   n_slots      device int32 [n_seq] compressed slots per sequence
 *   max_slots    host bound on every n_vis (row stride of scores)
 *   scores       device fp32 [n_q][max_slots]; entries s < n_vis(t) written
 */
slc_status_t slc_index_scores(int n_q, int h_idx, const uint8_t *q_fp8, const float *q_scale,
                              const float *w, const int32_t *q_seq, const int32_t *q_pos,
                              int ratio, slc_pool_t key_pool, const int32_t *n_slots,
                              int max_slots, float *scores, void *stream);

/*
 * slc_topk_select -- "DeepSeek-V4 attention layer types", Indexer / C4A
 * branch (global top-k per query).  For each query t, the min(k, n_vis(t))
 * slots with the largest scores (ties to the lower slot index; -0.0 equals
 * +0.0), written to topk_idx[t][0 .. len) in increasing slot order, the rest
 * of the row set to -1; topk_len[t] = min(k, n_vis(t)).
 *
 *   scores       device fp32 [n_q][max_slots] (as written by slc_index_scores)
 *   k            1 .. SLC_MAX_TOPK
 *   topk_idx     device int32 [n_q][k];  topk_len  device int32 [n_q]
 */
slc_status_t slc_topk_select(int n_q, int k, const float *scores, int max_slots,
                             const int32_t *q_seq, const int32_t *q_pos, int ratio,
                             const int32_t *n_slots, int32_t *topk_idx, int32_t *topk_len,
                             void *stream);

/*
 * slc_topk_select_warm -- slc_topk_select, plus an L2 warm-up for the sparse
 * MLA decode that follows it: spare workgroups of the same launch read, and
 * discard, each query's inputs that do not depend on the selection (its
 * query heads q[t][0..n_heads) and the latent rows of its window, the
 * positions max(0, p-window+1) .. p of swa_pool), so that the decode finds
 * them in cache.  The select uses one compute unit per query, so these
 * reads run beside it.  Outputs are identical to slc_topk_select's.
 *   q, n_heads, window, swa_pool  as for slc_sparse_mla_decode (q 16-byte
 *                                 aligned; swa_pool required when window > 0)
 *   ratio        as for slc_topk_select, OR'ed with SLC_SWA_FP8 when swa_pool
 *                holds fp8 rows (CMP layout)
 */
slc_status_t slc_topk_select_warm(int n_q, int k, const float *scores, int max_slots,
                                  const int32_t *q_seq, const int32_t *q_pos, int ratio,
                                  const int32_t *n_slots, int32_t *topk_idx, int32_t *topk_len,
                                  const uint16_t *q, int n_heads, int window, slc_pool_t swa_pool,
                                  void *stream);

/* Bytes of workspace slc_index_topk needs: the fp32 scores of every visible
 * slot, [n_q][max_slots], which the select reads back.  Host arithmetic only;
 * 0 when n_q or max_slots is not positive.  The pages size such scratch on the
 * host before any real call ("DeepseekV4Attention" (devpress), forward_mqa:
 * the warm-up dummy run only allocates the workspace) and hand it to the
 * kernels from a workspace manager (_forward_prefill, step 3). */
size_t slc_index_topk_workspace_size(int n_q, int max_slots);

/* slc_index_scores followed by slc_topk_select, scores kept in `workspace`
 * (device, >= slc_index_topk_workspace_size bytes, 256-byte aligned); ratio
 * may carry SLC_KEY_MXFP4 as for slc_index_scores. */
slc_status_t slc_index_topk(int n_q, int h_idx, int k, const uint8_t *q_fp8,
                            const float *q_scale, const float *w, const int32_t *q_seq,
                            const int32_t *q_pos, int ratio, slc_pool_t key_pool,
                            const int32_t *n_slots, int max_slots, int32_t *topk_idx,
                            int32_t *topk_len, void *workspace, size_t ws_bytes, void *stream);

/*
 * slc_indexcache_skips -- "DeepSeek-V4 IndexCache freq2 cross-layer TopK
 * reuse" (the IndexCache freq2 page), section 2: which layers reuse an
 * earlier layer's top-k list instead of running the indexer and the select.
 * Only layers with compress ratio 4 take part.  A layer's sequence index is
 * the number of ratio-4 layers before it.  Without a pattern it reuses when
 * that index is not a multiple of freq (freq <= 1: never).  A non-empty
 * pattern takes priority: it must begin with 'F' and hold only 'F'
 * (compute) and 'S' (reuse), position i deciding for sequence index i;
 * layers past its end compute.  A reusing layer passes the list of the
 * layer that last computed one to its attention as a given top-k (the
 * compressor keeps running on every layer).
 *   n_layers         layers in the stack
 *   compress_ratios  HOST int32 [n_layers] (4 marks the indexed layers)
 *   freq             reuse frequency
 *   pattern          HOST, NUL-terminated, nullable or "" for none
 *   skip             HOST int32 [n_layers] out: 1 = reuse, 0 = compute
 * Host arithmetic only (no GPU).  Errors: SLC_ERR_INVALID_ARG for a bad
 * pattern or missing pointers.
 */
slc_status_t slc_indexcache_skips(int n_layers, const int32_t *compress_ratios, int freq,
                                  const char *pattern, int32_t *skip);

/*
 * slc_sparse_mla_decode / slc_sparse_mla_prefill -- "DeepseekV4Attention"
 * (devpress), forward_mqa with _forward_decode (flash_mla_with_kvcache with
 * SWA and compressed indices) and _forward_prefill (flash_mla_sparse_fwd over
 * top-k combined with SWA indices); "From MLA to CSA + HCA" Ch.2 (absorbed
 * MQA: H query heads against one shared 576-wide latent head).
 *
 * For query t (sequence b = q_seq[t], position p = q_pos[t]) the attended
 * list is, without deduplication,
 *   SWA: positions max(0, p-window+1) .. p, rows of swa_pool;
 *   CMP: cmp_idx[t][0..k) entries with 0 <= idx < n_slots[b] (others
 *        skipped), rows of cmp_pool dequantised as code * scale (exact in bf16)
 *        ++ the bf16 rope dims   [c4a, c128a only].
 *   logit_i = sm_scale * q[t][h] . K_i (576 dims)
 *   out[t][h] = sum_i softmax(logit)_i * K_i[0:512]  (bf16, round to nearest)
 *   lse[t][h] = ln sum_i exp(logit_i)  (fp32; -inf and out = 0 if the list is empty)
 *
 *   layer_type   SLC_LAYER_SWAONLY (cmp_pool, cmp_idx ignored; k must be 0),
 *                SLC_LAYER_C4A or SLC_LAYER_C128A (cmp_pool, cmp_idx required);
 *                OR'ed with SLC_SWA_FP8 when swa_pool holds fp8 rows in the
 *                CMP layout (dequantised like compressed rows; the SWA rows
 *                are then K_i = code * scale ++ rope as well)
 *   n_q, n_heads queries and query heads (multiple of 16, <= 128)
 *   q            device bf16 [n_q][n_heads][576], 16-byte aligned
 *   q_seq, q_pos device int32 [n_q]
 *   window       sliding-window length, 0 .. SLC_MAX_WINDOW
 *   cmp_idx      device int32 [n_q][k] logical slot ids (-1 = none)
 *   n_slots      device int32 [n_seq]
 *   out          device bf16 [n_q][n_heads][512], 16-byte aligned;
 *                lse nullable fp32 [n_q][n_heads]
 *   workspace    device, >= the matching *_workspace_size bytes, 256-B aligned
 * Decode splits each query's list across workgroups and merges the partial
 * softmax states; prefill gives each query token its own workgroup.  Both
 * compute the same function.
 */
/* Workspace sizes of the two attention calls (host arithmetic only, the
 * same sizing passages as slc_index_topk_workspace_size: "DeepseekV4Attention"
 * (devpress), forward_mqa's dummy run and _forward_prefill's workspace
 * manager).  Decode: the partial (O, max, sum) states of the list splits the
 * call's split plan forms for these shapes, 0 when it forms one split;
 * prefill: always 0 (one workgroup per query token, nothing to merge).
 * k is the compressed list length the call will pass (0 for SWAONLY). */
size_t slc_sparse_mla_decode_workspace_size(int n_q, int n_heads, int window, int k);
slc_status_t slc_sparse_mla_decode(int layer_type, int n_q, int n_heads, const uint16_t *q,
                                   const int32_t *q_seq, const int32_t *q_pos, int window,
                                   slc_pool_t swa_pool, slc_pool_t cmp_pool,
                                   const int32_t *cmp_idx, int k, const int32_t *n_slots,
                                   float sm_scale, uint16_t *out, float *lse, void *workspace,
                                   size_t ws_bytes, void *stream);

/*
 * slc_sparse_mla_decode_topk -- the C4A branch's top-k select and the decode
 * over its list in one call: "DeepSeek-V4 attention layer types", Indexer /
 * C4A branch (the indexer's global top-k per query feeds the compressed
 * indices of the attention) with "DeepseekV4Attention" (devpress),
 * _forward_decode (the SWA and the compressed indices go to one attention
 * kernel).  Results are those of slc_topk_select(k, scores, ...) followed by
 * slc_sparse_mla_decode(layer_type, ..., topk_idx, k, ...): the same list,
 * written to topk_idx / topk_len, and the same out / lse, bit for bit.
 * Where the shapes allow (scores 16-byte aligned, 4 <= max_slots <= 16384,
 * max_slots a multiple of 4, and the split plan's compressed share of a
 * split at most 512 entries) the decode's workgroups select the list
 * themselves in the same launch; otherwise the call runs the two steps.
 *
 *   layer_type   SLC_LAYER_C4A, optionally OR'ed with SLC_SWA_FP8
 *   k            1 .. SLC_MAX_TOPK; scores / max_slots as slc_topk_select
 *                (the visible count of query t is min(n_slots[q_seq[t]],
 *                (q_pos[t] + 1) / 4), at most max_slots)
 *   topk_idx     device int32 [n_q][k];  topk_len  device int32 [n_q]
 *   other arguments, the workspace and its size as slc_sparse_mla_decode
 *   (slc_sparse_mla_decode_workspace_size(n_q, n_heads, window, k)).
 */
slc_status_t slc_sparse_mla_decode_topk(int layer_type, int n_q, int n_heads, const uint16_t *q,
                                        const int32_t *q_seq, const int32_t *q_pos, int window,
                                        slc_pool_t swa_pool, slc_pool_t cmp_pool, int k,
                                        const float *scores, int max_slots,
                                        const int32_t *n_slots, int32_t *topk_idx,
                                        int32_t *topk_len, float sm_scale, uint16_t *out,
                                        float *lse, void *workspace, size_t ws_bytes,
                                        void *stream);

/*
 * slc_sparse_mla_decode_noalloc -- slc_sparse_mla_decode for callers that
 * cannot allocate device memory or pass a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * kernels and results; the split partials go to a static device array of
 * slc_sparse_mla_decode_noalloc_max_bytes() bytes (12 MiB) that the library
 * holds on each GPU it runs on until the process ends.  Its device address
 * is resolved on the first call on each device (with that device current).
 * The call allocates nothing (no hipMalloc, no library allocation).
 *   Arguments and results as slc_sparse_mla_decode, without the workspace.
 *   Shapes whose partials exceed the array (slc_sparse_mla_decode_workspace_size
 *   above the maximum) return SLC_ERR_WORKSPACE before any launch; the 64K
 *   decode (32 queries, 64 heads, window 128, top-k 512) needs about 8.5 MB;
 *   the split plan bounds any shape's partials by about 17 MB.
 *   Nothing in the array needs to start cleared: every partial is written
 *   before it is merged.  All calls on one GPU share the array, so calls that
 *   may overlap on one GPU (other streams, other host threads) race.
 */
size_t slc_sparse_mla_decode_noalloc_max_bytes(void);
slc_status_t slc_sparse_mla_decode_noalloc(int layer_type, int n_q, int n_heads,
                                           const uint16_t *q, const int32_t *q_seq,
                                           const int32_t *q_pos, int window, slc_pool_t swa_pool,
                                           slc_pool_t cmp_pool, const int32_t *cmp_idx, int k,
                                           const int32_t *n_slots, float sm_scale, uint16_t *out,
                                           float *lse, void *stream);

size_t slc_sparse_mla_prefill_workspace_size(int n_q, int n_heads, int window, int k);
slc_status_t slc_sparse_mla_prefill(int layer_type, int n_q, int n_heads, const uint16_t *q,
                                    const int32_t *q_seq, const int32_t *q_pos, int window,
                                    slc_pool_t swa_pool, slc_pool_t cmp_pool,
                                    const int32_t *cmp_idx, int k, const int32_t *n_slots,
                                    float sm_scale, uint16_t *out, float *lse, void *workspace,
                                    size_t ws_bytes, void *stream);

/*
 * slc_workspace_size -- one sizer for every call that takes a workspace.
 * "DeepseekV4Attention" (devpress), forward_mqa: the warm-up dummy run does
 * nothing but allocate the workspace, so the size must follow from the
 * shapes alone, before any real call; _forward_prefill (step 3) then takes
 * its scratch from the workspace manager rather than allocating per call.
 * This library keeps the same split: the caller sizes and owns the
 * workspace, the calls only use it.
 *
 *   op      SLC_OP_INDEX_TOPK          slc_index_topk (uses n_q, max_slots)
 *           SLC_OP_SPARSE_MLA_DECODE   slc_sparse_mla_decode (n_q, n_heads,
 *                                      window, k)
 *           SLC_OP_SPARSE_MLA_PREFILL  slc_sparse_mla_prefill (the same)
 *   shape   HOST pointer; fields an op does not use are ignored
 * Returns the bytes the call needs (0: it needs none; pass NULL), equal to
 * the matching per-op sizer's result.  An unknown op or a NULL shape returns
 * SIZE_MAX, which no allocation satisfies.  Host arithmetic only.
 */
typedef enum {
    SLC_OP_INDEX_TOPK = 1,
    SLC_OP_SPARSE_MLA_DECODE = 2,
    SLC_OP_SPARSE_MLA_PREFILL = 3
} slc_op_t;

typedef struct slc_shape {
    int n_q;         /* queries: sequences (decode) or tokens (prefill, index) */
    int n_heads;     /* query heads (attention)                               */
    int window;      /* sliding-window length (attention)                     */
    int k;           /* top-k / compressed list length                        */
    int max_slots;   /* index: row stride of the scores                       */
} slc_shape_t;

size_t slc_workspace_size(slc_op_t op, const slc_shape_t *shape);

#ifdef __cplusplus
}
#endif

#endif /* SLC_H */
