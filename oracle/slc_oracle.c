/*
 * slc_oracle.c -- plain, slow CPU oracle for one compressed sparse attention
 * layer (DeepSeek-V4 style: compressor, lightning indexer + top-k, sparse MLA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under sparse_long_context_compressor_amd/) never calls it, and
 * the two share no source: no headers, helpers, tables or constants.
 *
 * Everything here works on *logical* per-sequence arrays in host memory (no
 * paging); floating point is evaluated in double and rounded once to the
 * output format.  Where floating point decides an integer (an fp8 code, a
 * top-k membership) the decision is taken on the fp32 value, the precision
 * the compressor state and the indexer accumulate in on the pages.
 *
 * Sources (the pages' titles; sections named as on each page):
 *  [P1] "DeepSeek V4 attention in vLLM" (juejin.cn post 7667401749827403791):
 *       layer-type table; "Compressor: ratio 4 vs 128" (window diagram,
 *       position rule (pos//r)*r, start-of-sequence masking); "Indexer, C4A
 *       and C128A top-k branch".
 *  [P3] "DeepseekV4Attention" (devpress.csdn.net, AMD): DeepseekCompressor
 *       forward (RoPE conventions), "CSA compressor" (softmax-gated pooling
 *       formula, boundary table), "Indexer" (I_{t,s} formula), cache block
 *       layout (fp8 nope + bf16 rope + per-64 scales).
 *  [P5] "DeepSeek attention evolution: MLA to CSA/HCA": 5.1 CSA (slot j
 *       covers [4j-4, 4j+3], anchor 4j, causality i >= 4j+3), 5.2 HCA
 *       ([128j, 128j+127]), 6.1 (fp8 e4m3 + UE8M0 scales), 6.3 (slot
 *       mapping: valid iff (pos+1) % r == 0, slot = pos // r), Ch.2 MLA
 *       (absorbed MQA over the 576-wide latent, values = first 512 dims).
 *
 * Readings taken where the pages are silent or disagree: slots are
 * ceil(L/r) with a trailing partial slot pooled
 * over the tokens present; softmax is per channel over the window's tokens;
 * RMSNorm runs over all 576 latent dims; the pow2 scale is the smallest 2^e
 * with amax <= 448 * 2^e (exact comparison), stored as fp32; fp8 is OCP
 * E4M3FN with round-to-nearest-even; top-k ties go to the lower slot index;
 * the streaming compressor's older token group brings block 0 (C_a) and the
 * newer block 1 (C_b); MXFP4 keys put the even element in the low nibble and
 * scale each 32-dim block by the smallest 2^e with amax <= 6 * 2^e.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_pins.py
 * (closed forms, worked examples from the pages, library routines for the
 * codecs, brute force over the full pool); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_D 576      /* latent row: 512 nope + 64 rope            [P5 Ch.2] */
#define OR_DN 512     /* value / nope width                        [P5 Ch.2] */
#define OR_DR 64      /* rope width                                [P3]      */
#define OR_QB 64      /* fp8 quantisation block                    [P5 6.1]  */
#define OR_DI 128     /* indexer head dim                          [P3]      */
#define OR_E4M3_MAX 448.0

/* ------------------------------------------------------------------ codecs */

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * S.1111.111 is NaN; largest finite 448 = 1.75 * 2^8. */
double oracle_e4m3_value(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);          /* m/8 * 2^(1-7) */
    else
        v = ldexp(8.0 + m, e - 10);        /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* Round x to the nearest E4M3FN value, ties to even; magnitudes at or above
 * 448 saturate to 448.  The sign of a value that rounds to zero is kept. */
uint8_t oracle_e4m3_encode(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x), quantum, v;
    int ex, lg;
    if (isnan(x))
        return 0x7F;
    if (a >= OR_E4M3_MAX)
        return sign | 0x7E;
    if (a == 0.0)
        return sign;
    frexp(a, &ex);                 /* a = f * 2^ex, f in [0.5, 1) */
    lg = ex - 1;                   /* floor(log2 a) */
    if (lg < -6)
        lg = -6;                   /* subnormal range shares 2^-6's quantum */
    quantum = ldexp(1.0, lg - 3);  /* 3 mantissa bits */
    v = nearbyint(a / quantum) * quantum;   /* default mode: ties to even */
    if (v == 0.0)
        return sign;
    frexp(v, &ex);
    lg = ex - 1;
    if (lg < -6)
        return sign | (uint8_t)(v * 512.0);            /* subnormal: v / 2^-9 */
    return sign | (uint8_t)(((lg + 7) << 3) | ((int)ldexp(v, 3 - lg) - 8));
}

double oracle_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round x to the nearest bfloat16 (8 significant bits, fp32 exponent range),
 * ties to even, overflow to infinity. */
uint16_t oracle_bf16_encode(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    double a = fabs(x), quantum, v;
    int ex, lg;
    float f;
    uint32_t u;
    if (isnan(x))
        return 0x7FC0;
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    frexp(a, &ex);
    lg = ex - 1;
    if (lg < -126)
        lg = -126;                 /* subnormal quantum is 2^-133 */
    quantum = ldexp(1.0, lg - 7);
    v = nearbyint(a / quantum) * quantum;
    if (v >= ldexp(1.0, 128))
        return sign | 0x7F80;
    f = (float)v;                  /* exact: v has <= 8 significant bits */
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------ slot algebra */

/* Slots a sequence of L tokens produces: ceil(L / r).  The pages emit a slot
 * when (pos+1) % r == 0 [P5 6.3], i.e. floor(L/r) complete slots; a trailing
 * partial window is also pooled (over the tokens present) but no query inside
 * the sequence can see it (oracle_n_visible). */
int oracle_n_slots(int L, int r)
{
    return L <= 0 ? 0 : (L + r - 1) / r;
}

/* Slots visible to a query at position p: j with p >= r*j + r - 1 [P5 5.1],
 * capped by the slots that exist. */
int oracle_n_visible(int p, int r, int n_slots)
{
    int v = (p + 1) / r;
    if (v > n_slots)
        v = n_slots;
    return v < 0 ? 0 : v;
}

/* Token window of slot j: r=4 gathers 2r tokens with stride r, covering
 * [4j-4, 4j+3] [P5 5.1; P3 boundary table]; r=128 covers [128j, 128j+127]
 * [P5 5.2].  Clipped to [0, L) [P1: the first window only uses pos >= 0]. */
void oracle_window(int j, int r, int L, int *t_lo, int *t_hi)
{
    int coff = (r == 4) ? 2 : 1;
    int lo = r * j - (coff - 1) * r, hi = r * j + r - 1;
    *t_lo = lo < 0 ? 0 : lo;
    *t_hi = hi > L - 1 ? L - 1 : hi;
}

/* --------------------------------------------------------------- compress */

static int pow2_exponent_for(double amax)
{
    int ex, e;
    if (amax == 0.0)
        return 0;
    frexp(amax / OR_E4M3_MAX, &ex);
    e = ex;
    while (amax <= ldexp(OR_E4M3_MAX, e - 1))
        e--;
    while (amax > ldexp(OR_E4M3_MAX, e))
        e++;
    /* the scale is stored as an fp32 power of two: below 2^-126 it would no
     * longer be a normal fp32, so tinier blocks share that scale (their codes
     * round toward zero) */
    return e < -126 ? -126 : e;
}

/* The cache row format ["DeepseekV4Attention", cache block layout; "From
 * MLA to CSA + HCA" 6.1]: the 512 nope dims of the fp32 row y32 in 8 blocks of
 * 64, each with the pow2 scale of its largest magnitude and e4m3 codes of
 * y / scale (round to nearest even); the 64 rope dims rounded to bf16. */
static void quantise_row(const float *y32, uint8_t *codes, float *scales, uint16_t *rope)
{
    for (int blk = 0; blk < OR_DN / OR_QB; blk++) {
        double amax = 0.0, scale;
        for (int i = 0; i < OR_QB; i++) {
            double a = fabs((double)y32[blk * OR_QB + i]);
            if (a > amax)
                amax = a;
        }
        scale = ldexp(1.0, pow2_exponent_for(amax));
        scales[blk] = (float)scale;
        for (int i = 0; i < OR_QB; i++)
            codes[blk * OR_QB + i] = oracle_e4m3_encode((double)y32[blk * OR_QB + i] / scale);
    }
    for (int i = 0; i < OR_DR; i++)
        rope[i] = oracle_bf16_encode((double)y32[OR_DN + i]);
}

/* The steps after the pool [P3 CSA compressor diagram; P5 6.2]: RMSNorm over
 * the 576 dims, RoPE on the pairs (512+2i, 513+2i) at position pos, the row
 * rounded to fp32, then the cache row format.  -1 if pos is past the table. */
static int finish_slot(const double *pooled, int pos, const float *gamma, double eps,
                       const float *cos_sin, int max_pos, uint8_t *codes, float *scales,
                       uint16_t *rope, float *prequant_out)
{
    double y[OR_D], ms = 0.0, inv;
    float y32[OR_D];
    for (int d = 0; d < OR_D; d++)
        ms += pooled[d] * pooled[d];
    ms /= OR_D;
    inv = 1.0 / sqrt(ms + eps);
    for (int d = 0; d < OR_D; d++)
        y[d] = pooled[d] * inv * (double)gamma[d];
    if (pos >= max_pos)
        return -1;
    for (int i = 0; i < OR_DR / 2; i++) {
        double c = cos_sin[(size_t)pos * OR_DR + i];
        double s = cos_sin[(size_t)pos * OR_DR + OR_DR / 2 + i];
        double a = y[OR_DN + 2 * i], b = y[OR_DN + 2 * i + 1];
        y[OR_DN + 2 * i] = a * c - b * s;
        y[OR_DN + 2 * i + 1] = a * s + b * c;
    }
    for (int d = 0; d < OR_D; d++)
        y32[d] = (float)y[d];
    if (prequant_out)
        memcpy(prequant_out, y32, sizeof y32);
    quantise_row(y32, codes, scales, rope);
    return 0;
}

/*
 * One sequence of L tokens, ratio r in {4, 128}.
 *   kv    [L, 576] bf16 bits     per-token latent kv
 *   score [L, 576] fp32          per-token gate logits (post-APE)
 *   gamma [576] fp32, eps        RMSNorm weight
 *   cos_sin [max_pos, 64] fp32   row p: 32 cos then 32 sin
 * Outputs for each of n = ceil(L/r) slots:
 *   codes [n, 512] e4m3, scales [n, 8] fp32 (powers of two), rope [n, 64] bf16;
 *   pooled [n, 576] double (nullable) -- the softmax-pooled row;
 *   prequant [n, 576] fp32 (nullable) -- the row after RMSNorm and RoPE.
 * Returns 0, or -1 when a slot's anchor position is outside the table.
 *
 * Steps, in the pages' order [P3 CSA compressor diagram; P5 6.2]:
 *  pool:  per channel d, w_t = softmax over t in the window of score[t][d];
 *         pooled[d] = sum_t w_t kv[t][d]                       [P3; P5 5.1]
 *  norm:  y = pooled * gamma / sqrt(mean(pooled^2) + eps)       [P3]
 *  rope:  GPT-J interleaved pairs (512+2i, 513+2i) of the last 64 dims,
 *         at position (pos // r) * r = r*j, cos/sin from the table [P3, P1]
 *  quant: nope dims in 8 blocks of 64 -> e4m3 codes + pow2 scale;
 *         rope dims -> bf16                                    [P3; P5 6.1]
 */
int oracle_compress_seq(int r, int L, const uint16_t *kv, const float *score,
                        const float *gamma, double eps, const float *cos_sin,
                        int max_pos, uint8_t *codes, float *scales,
                        uint16_t *rope, double *pooled_out, float *prequant_out)
{
    int n = oracle_n_slots(L, r);
    for (int j = 0; j < n; j++) {
        double pooled[OR_D];
        int t_lo, t_hi;

        oracle_window(j, r, L, &t_lo, &t_hi);
        for (int d = 0; d < OR_D; d++) {
            double m = -INFINITY, se = 0.0, acc = 0.0;
            for (int t = t_lo; t <= t_hi; t++)
                if ((double)score[(size_t)t * OR_D + d] > m)
                    m = score[(size_t)t * OR_D + d];
            for (int t = t_lo; t <= t_hi; t++) {
                double e = exp((double)score[(size_t)t * OR_D + d] - m);
                se += e;
                acc += e * oracle_bf16_value(kv[(size_t)t * OR_D + d]);
            }
            pooled[d] = acc / se;
        }
        if (pooled_out)
            memcpy(pooled_out + (size_t)j * OR_D, pooled, sizeof pooled);
        if (finish_slot(pooled, r * j, gamma, eps, cos_sin, max_pos, codes + (size_t)j * OR_DN,
                        scales + (size_t)j * (OR_DN / OR_QB), rope + (size_t)j * OR_DR,
                        prequant_out ? prequant_out + (size_t)j * OR_D : NULL))
            return -1;
    }
    return 0;
}

/*
 * Streaming compressor, in its two-block form ["DeepseekV4Attention",
 * DeepseekCompressor forward (save_partial_states adds the APE bias to the
 * scores and keeps kv and score in an fp32 state cache) and "CSA compressor"
 * (the C_a / C_b formula and the state layout table); "From MLA to CSA +
 * HCA" 5.5 (a slot is compressed once its last token arrives)].
 *   kv    [L, coff*576] bf16 bits: each token's coff kv blocks (r = 4: C_a
 *         then C_b, coff = 2; r = 128: one block, coff = 1)
 *   score [L, coff*576] fp32: the matching gate blocks (Z_a, Z_b)
 *   ape   [r, coff*576] fp32: the positional bias (B_a, B_b), row pos % r
 * Slot j is emitted when token r*j + r - 1 has arrived: slots j < floor(L/r).
 * Its window entries, per channel d:
 *   r = 4:   tokens 4j-4 .. 4j-1 (those >= 0) with their block 0 (C_a),
 *            tokens 4j .. 4j+3 with their block 1 (C_b);
 *   r = 128: tokens 128j .. 128j+127 with block 0.
 * An entry's logit is the fp32 state value fp32(score + ape) and its value
 * the kv block's; the pool is the per-channel softmax-weighted sum, then
 * RMSNorm, RoPE at r*j and quantisation exactly as oracle_compress_seq.
 * Outputs as oracle_compress_seq for the floor(L/r) emitted slots.
 * Returns 0, or -1 when a slot's anchor is outside the cos/sin table.
 */
int oracle_compress_stream_seq(int r, int L, const uint16_t *kv, const float *score,
                               const float *ape, const float *gamma, double eps,
                               const float *cos_sin, int max_pos, uint8_t *codes,
                               float *scales, uint16_t *rope, float *prequant_out)
{
    int coff = r == 4 ? 2 : 1, w = coff * OR_D;
    int n = L / r;
    for (int j = 0; j < n; j++) {
        double pooled[OR_D];
        int t_lo = r * j - (coff - 1) * r, t_hi = r * j + r - 1;
        if (t_lo < 0)
            t_lo = 0;
        for (int d = 0; d < OR_D; d++) {
            double m = -INFINITY, se = 0.0, acc = 0.0;
            for (int pass = 0; pass < 2; pass++) {
                for (int t = t_lo; t <= t_hi; t++) {
                    int blk = (coff == 2 && t >= r * j) ? 1 : 0;
                    size_t c = (size_t)t * w + (size_t)blk * OR_D + d;
                    double logit = (float)(score[c] + ape[(size_t)(t % r) * w + blk * OR_D + d]);
                    if (pass == 0) {
                        if (logit > m)
                            m = logit;
                    } else {
                        double e = exp(logit - m);
                        se += e;
                        acc += e * oracle_bf16_value(kv[c]);
                    }
                }
            }
            pooled[d] = acc / se;
        }
        if (finish_slot(pooled, r * j, gamma, eps, cos_sin, max_pos, codes + (size_t)j * OR_DN,
                        scales + (size_t)j * (OR_DN / OR_QB), rope + (size_t)j * OR_DR,
                        prequant_out ? prequant_out + (size_t)j * OR_D : NULL))
            return -1;
    }
    return 0;
}

/*
 * SWA KV insert ["From MLA to CSA + HCA" 6.2: the fused q-norm / RoPE / KV
 * insert kernel's KV side (GPT-J RoPE, fp8 quantisation, paged write); 5.5:
 * the SWA cache holds fp8 nope + bf16 rope + one scale per 64 dims;
 * "DeepseekV4Attention", HCA compressor workflow stage 3 (KV: RoPE + FP8
 * quant + SWA cache write)].
 *   kv [n, 576] bf16 bits: the tokens' latent rows, not yet rotated
 *   pos [n]: each token's own position (row of the cos/sin table)
 * Each row: RoPE on the pairs (512+2i, 513+2i) at pos, the row rounded to
 * fp32, then the compressed rows' quantisation (codes [n,512], scales [n,8],
 * rope [n,64]); prequant [n,576] (nullable) receives the fp32 row.
 * Returns 0, or -1 when a position is outside the table (nothing after that
 * token is written).
 */
int oracle_swa_insert(int n, const uint16_t *kv, const int32_t *pos, const float *cos_sin,
                      int max_pos, uint8_t *codes, float *scales, uint16_t *rope,
                      float *prequant_out)
{
    for (int t = 0; t < n; t++) {
        double y[OR_D];
        float y32[OR_D];
        int p = pos[t];
        if (p < 0 || p >= max_pos)
            return -1;
        for (int d = 0; d < OR_D; d++)
            y[d] = oracle_bf16_value(kv[(size_t)t * OR_D + d]);
        for (int i = 0; i < OR_DR / 2; i++) {
            double c = cos_sin[(size_t)p * OR_DR + i];
            double s = cos_sin[(size_t)p * OR_DR + OR_DR / 2 + i];
            double a = y[OR_DN + 2 * i], b = y[OR_DN + 2 * i + 1];
            y[OR_DN + 2 * i] = a * c - b * s;
            y[OR_DN + 2 * i + 1] = a * s + b * c;
        }
        for (int d = 0; d < OR_D; d++)
            y32[d] = (float)y[d];
        if (prequant_out)
            memcpy(prequant_out + (size_t)t * OR_D, y32, sizeof y32);
        quantise_row(y32, codes + (size_t)t * OR_DN, scales + (size_t)t * (OR_DN / OR_QB),
                     rope + (size_t)t * OR_DR);
    }
    return 0;
}

/* Several sequences packed back to back: cu_seqlens [n_seq+1] token offsets;
 * slot outputs packed the same way with cu_slots[b] = sum of ceil(L_b'/r)
 * over earlier sequences.  Returns 0 or the first failing sequence's -1. */
int oracle_compress_batch(int r, int n_seq, const int32_t *cu_seqlens,
                          const uint16_t *kv, const float *score,
                          const float *gamma, double eps, const float *cos_sin,
                          int max_pos, uint8_t *codes, float *scales,
                          uint16_t *rope, float *prequant_out)
{
    int rc = 0;
    int64_t slot0 = 0;
    for (int b = 0; b < n_seq; b++) {
        int L = cu_seqlens[b + 1] - cu_seqlens[b];
        size_t t0 = (size_t)cu_seqlens[b];
        if (oracle_compress_seq(r, L, kv + t0 * OR_D, score + t0 * OR_D, gamma,
                                eps, cos_sin, max_pos, codes + slot0 * OR_DN,
                                scales + slot0 * (OR_DN / OR_QB),
                                rope + slot0 * OR_DR, NULL,
                                prequant_out ? prequant_out + slot0 * OR_D : NULL))
            rc = -1;
        slot0 += oracle_n_slots(L, r);
    }
    return rc;
}

/* ---------------------------------------------------------------- indexer */

/*
 * Lightning-indexer scores of one query against n keys [P3 Indexer]:
 *   I_s = sum_j w_j * ReLU(q_j . k_s),  with the fp8 dequantisation scales
 *   folded in: q_j . k_s = q_scale_j * k_scale_s * sum_d q_j[d] k_s[d].
 * The fp8 dot is exact in double (each product is an integer multiple of
 * 2^-18 below 2^18, and 128 of them stay below 2^53).  out64 is the double
 * value, out32 its fp32 rounding (the value top-k decides on).
 */
void oracle_index_scores(int h_idx, int n, const uint8_t *q, const float *q_scale,
                         const float *w, const uint8_t *keys,
                         const float *key_scale, float *out32, double *out64)
{
    double qv[OR_DI];
    double *acc = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    for (int j = 0; j < h_idx; j++) {
        for (int d = 0; d < OR_DI; d++)
            qv[d] = oracle_e4m3_value(q[(size_t)j * OR_DI + d]);
        for (int s = 0; s < n; s++) {
            double dot = 0.0, v;
            for (int d = 0; d < OR_DI; d++)
                dot += qv[d] * oracle_e4m3_value(keys[(size_t)s * OR_DI + d]);
            v = (double)q_scale[j] * (double)key_scale[s] * dot;
            if (v < 0.0)
                v = 0.0;
            acc[s] += (double)w[j] * v;
        }
    }
    for (int s = 0; s < n; s++) {
        if (out64)
            out64[s] = acc[s];
        if (out32)
            out32[s] = (float)acc[s];
    }
    free(acc);
}

/*
 * The indexer's own compressor ["DeepSeek-V4 attention layer types": the
 * indexer holds a small compressor of head_dim 128 whose entries fill the
 * indexer's K cache; "DeepseekV4Attention": the same compressor class (its
 * RoPE on the last 64 dims, at (pos // r) * r) and the indexer cache entry
 * of 128 fp8 values plus one fp32 scale].  Ratio 4, streamed in the
 * two-block form of oracle_compress_stream_seq with rows of 128 dims:
 *   kv, score [L, 2*128] (bf16 bits, fp32), ape [4, 2*128], gamma [128];
 * slot j pools positions 4j-4 .. 4j-1 (block 0) and 4j .. 4j+3 (block 1)
 * per channel, then RMSNorm over the 128 dims, RoPE on the pairs
 * (64+2i, 65+2i) at position 4j, the row rounded to fp32, and one pow2 scale
 * for all 128 dims (the compressed rows' rule) with e4m3 codes of y / scale.
 * Outputs for the floor(L/4) emitted slots: codes [n,128], scales [n],
 * prequant [n,128] (nullable).  Returns -1 if an anchor is past the table.
 */
int oracle_compress_index_keys_stream_seq(int L, const uint16_t *kv, const float *score,
                                          const float *ape, const float *gamma, double eps,
                                          const float *cos_sin, int max_pos, uint8_t *codes,
                                          float *scales, float *prequant_out)
{
    const int r = 4, w = 2 * OR_DI;
    int n = L / r;
    for (int j = 0; j < n; j++) {
        double pooled[OR_DI], y[OR_DI], ms = 0.0, inv, amax = 0.0, scale;
        float y32[OR_DI];
        int t_lo = r * j - r < 0 ? 0 : r * j - r, t_hi = r * j + r - 1, pos = r * j;
        for (int d = 0; d < OR_DI; d++) {
            double m = -INFINITY, se = 0.0, acc = 0.0;
            for (int pass = 0; pass < 2; pass++) {
                for (int t = t_lo; t <= t_hi; t++) {
                    int blk = t >= r * j ? 1 : 0;
                    size_t c = (size_t)t * w + (size_t)blk * OR_DI + d;
                    double logit = (float)(score[c] + ape[(size_t)(t % r) * w + blk * OR_DI + d]);
                    if (pass == 0) {
                        if (logit > m)
                            m = logit;
                    } else {
                        double e = exp(logit - m);
                        se += e;
                        acc += e * oracle_bf16_value(kv[c]);
                    }
                }
            }
            pooled[d] = acc / se;
        }
        for (int d = 0; d < OR_DI; d++)
            ms += pooled[d] * pooled[d];
        ms /= OR_DI;
        inv = 1.0 / sqrt(ms + eps);
        for (int d = 0; d < OR_DI; d++)
            y[d] = pooled[d] * inv * (double)gamma[d];
        if (pos >= max_pos)
            return -1;
        for (int i = 0; i < OR_DR / 2; i++) {
            double c = cos_sin[(size_t)pos * OR_DR + i];
            double s = cos_sin[(size_t)pos * OR_DR + OR_DR / 2 + i];
            double a = y[OR_DI - OR_DR + 2 * i], b = y[OR_DI - OR_DR + 2 * i + 1];
            y[OR_DI - OR_DR + 2 * i] = a * c - b * s;
            y[OR_DI - OR_DR + 2 * i + 1] = a * s + b * c;
        }
        for (int d = 0; d < OR_DI; d++) {
            y32[d] = (float)y[d];
            if (fabs((double)y32[d]) > amax)
                amax = fabs((double)y32[d]);
        }
        if (prequant_out)
            memcpy(prequant_out + (size_t)j * OR_DI, y32, sizeof y32);
        scale = ldexp(1.0, pow2_exponent_for(amax));
        scales[j] = (float)scale;
        for (int d = 0; d < OR_DI; d++)
            codes[(size_t)j * OR_DI + d] = oracle_e4m3_encode((double)y32[d] / scale);
    }
    return 0;
}

/* ------------------------------------------------------- MXFP4 index keys */

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; no inf or NaN;
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 [P5 6.1: FP4 / MXFP4 indexer K
 * cache]. */
double oracle_e2m1_value(uint8_t nibble)
{
    int sign = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* Nearest e2m1 code of x, ties to the even code; magnitudes above 6 take 6. */
static uint8_t e2m1_encode(double x)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double a = fabs(x);
    int best = 0;
    for (int c = 1; c < 8; c++) {
        double dc = fabs(a - mag[c]), db = fabs(a - mag[best]);
        if (dc < db || (dc == db && (c & 1) == 0))
            best = c;
    }
    return (uint8_t)(best | (x < 0.0 ? 8 : 0));
}

/*
 * MXFP4 quantisation of index keys [P5 6.1: the FP4 / MXFP4 indexer K cache;
 * the OCP MX element and scale formats]: per 32-dim block, the scale is the
 * smallest 2^e with amax <= 6 * 2^e (1 if amax = 0; the same rule as the
 * fp8 rows with e2m1's largest magnitude 6), stored as the E8M0 byte e + 127,
 * and each element becomes the nearest e2m1 code of y / 2^e (ties to even),
 * two per byte with the even element in the low nibble.
 *   y [n, 128] fp32 -> codes4 [n, 64], e8m0 [n, 4].
 */
void oracle_mxfp4_quantise(int n, const float *y, uint8_t *codes4, uint8_t *e8m0)
{
    for (int s = 0; s < n; s++) {
        for (int b = 0; b < OR_DI / 32; b++) {
            double amax = 0.0, scale;
            int e = 0;
            for (int i = 0; i < 32; i++) {
                double a = fabs((double)y[(size_t)s * OR_DI + 32 * b + i]);
                if (a > amax)
                    amax = a;
            }
            if (amax > 0.0) {
                frexp(amax / 6.0, &e);
                while (amax <= ldexp(6.0, e - 1))
                    e--;
                while (amax > ldexp(6.0, e))
                    e++;
                if (e < -127)
                    e = -127;      /* E8M0's smallest scale, byte 0 = 2^-127 */
            }
            scale = ldexp(1.0, e);
            e8m0[(size_t)s * 4 + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; i += 2) {
                uint8_t lo = e2m1_encode((double)y[(size_t)s * OR_DI + 32 * b + i] / scale);
                uint8_t hi = e2m1_encode((double)y[(size_t)s * OR_DI + 32 * b + i + 1] / scale);
                codes4[(size_t)s * (OR_DI / 2) + 16 * b + i / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* OCP E8M0 block scale: 2^(byte - 127); 255 is NaN. */
double oracle_e8m0_value(uint8_t b)
{
    return b == 255 ? NAN : ldexp(1.0, (int)b - 127);
}

/*
 * Index scores against MXFP4 keys ["DeepseekV4Attention", Indexer: the FP4
 * indexer cache takes half the FP8 cache's bytes; "From MLA to CSA + HCA"
 * 6.1: FP4 / MXFP4 indexer keys; "DeepSeek-V4 attention layer types": the
 * FP4 indexer cache option]: key s holds 128 e2m1 values, two per byte (the
 * even element in the low nibble), keys4 [n, 64], and one E8M0 scale per 32
 * dims, key_e8m0 [n, 4].  Element d of the key is e2m1 * 2^(e - 127) of its
 * block, so the block scales sit inside the dot product:
 *   I[s] = sum_j w[j] * max(0, q_scale[j] * sum_d q[j][d] * k[s][d]).
 * Evaluated in double (the query side as in oracle_index_scores).
 */
void oracle_index_scores_mxfp4(int h_idx, int n, const uint8_t *q, const float *q_scale,
                               const float *w, const uint8_t *keys4,
                               const uint8_t *key_e8m0, float *out32, double *out64)
{
    double qv[OR_DI], kv[OR_DI];
    double *acc = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    for (int s = 0; s < n; s++) {
        for (int d = 0; d < OR_DI; d++) {
            uint8_t byte = keys4[(size_t)s * (OR_DI / 2) + d / 2];
            uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
            kv[d] = oracle_e2m1_value(nib) *
                    oracle_e8m0_value(key_e8m0[(size_t)s * (OR_DI / 32) + d / 32]);
        }
        for (int j = 0; j < h_idx; j++) {
            double dot = 0.0, v;
            for (int d = 0; d < OR_DI; d++) {
                qv[d] = oracle_e4m3_value(q[(size_t)j * OR_DI + d]);
                dot += qv[d] * kv[d];
            }
            v = (double)q_scale[j] * dot;
            if (v < 0.0)
                v = 0.0;
            acc[s] += (double)w[j] * v;
        }
    }
    for (int s = 0; s < n; s++) {
        if (out64)
            out64[s] = acc[s];
        if (out32)
            out32[s] = (float)acc[s];
    }
    free(acc);
}

struct or_pair { float v; int32_t i; };

static int cmp_score_desc_index_asc(const void *pa, const void *pb)
{
    const struct or_pair *a = (const struct or_pair *)pa, *b = (const struct or_pair *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/* Per-query global top-k [P1 C4A branch; P3 SparseAttnIndexer]: the min(k, n)
 * indices with the largest scores, ties to the lower index, listed in
 * (score desc, index asc) order and padded with -1 [P2: -1 fill].
 * Returns the length min(k, n). */
int oracle_topk(int n, const float *scores, int k, int32_t *idx)
{
    struct or_pair *p = (struct or_pair *)malloc(sizeof(struct or_pair) * (size_t)(n > 0 ? n : 1));
    int len = n < k ? n : k;
    for (int s = 0; s < n; s++) {
        p[s].v = scores[s];
        p[s].i = s;
    }
    qsort(p, (size_t)n, sizeof(struct or_pair), cmp_score_desc_index_asc);
    for (int t = 0; t < k; t++)
        idx[t] = t < len ? p[t].i : -1;
    free(p);
    return len;
}

/*
 * Scores + top-k for n_q queries.  Query t belongs to sequence q_seq[t] and
 * sits at position q_pos[t]; it scores the visible slots
 * s < n_visible(q_pos, r, n_slots[seq]).  Sequence b's keys start at key row
 * key_off[b] of keys [*, 128] e4m3 / key_scale [*].
 *   q [n_q, h_idx, 128] e4m3, q_scale / w [n_q, h_idx] fp32
 *   idx [n_q, k] int32 out, len [n_q] out
 *   scores32 [n_q, max_slots] fp32 out (nullable; unscored tail untouched)
 */
void oracle_index_topk_batch(int n_q, int h_idx, int k, const uint8_t *q,
                             const float *q_scale, const float *w,
                             const int32_t *q_pos, const int32_t *q_seq, int r,
                             const int64_t *key_off, const int32_t *n_slots,
                             const uint8_t *keys, const float *key_scale,
                             int32_t *idx, int32_t *len, float *scores32,
                             int max_slots)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < n_q; t++) {
        int b = q_seq[t];
        int nv = oracle_n_visible(q_pos[t], r, n_slots[b]);
        float *sc = (float *)malloc(sizeof(float) * (size_t)(nv > 0 ? nv : 1));
        oracle_index_scores(h_idx, nv, q + (size_t)t * h_idx * OR_DI,
                            q_scale + (size_t)t * h_idx, w + (size_t)t * h_idx,
                            keys + (size_t)key_off[b] * OR_DI,
                            key_scale + key_off[b], sc, NULL);
        len[t] = oracle_topk(nv, sc, k, idx + (size_t)t * k);
        if (scores32)
            memcpy(scores32 + (size_t)t * max_slots, sc, sizeof(float) * (size_t)nv);
        free(sc);
    }
}

/* The batch form of index top-k over MXFP4 keys: as oracle_index_topk_batch,
 * keys4 [.., 64] and key_e8m0 [.., 4] indexed from key_off[b]. */
void oracle_index_topk_batch_mxfp4(int n_q, int h_idx, int k, const uint8_t *q,
                                   const float *q_scale, const float *w,
                                   const int32_t *q_pos, const int32_t *q_seq, int r,
                                   const int64_t *key_off, const int32_t *n_slots,
                                   const uint8_t *keys4, const uint8_t *key_e8m0,
                                   int32_t *idx, int32_t *len, float *scores32, int max_slots)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < n_q; t++) {
        int b = q_seq[t];
        int nv = oracle_n_visible(q_pos[t], r, n_slots[b]);
        float *sc = (float *)malloc(sizeof(float) * (size_t)(nv > 0 ? nv : 1));
        oracle_index_scores_mxfp4(h_idx, nv, q + (size_t)t * h_idx * OR_DI,
                                  q_scale + (size_t)t * h_idx, w + (size_t)t * h_idx,
                                  keys4 + (size_t)key_off[b] * (OR_DI / 2),
                                  key_e8m0 + (size_t)key_off[b] * (OR_DI / 32), sc, NULL);
        len[t] = oracle_topk(nv, sc, k, idx + (size_t)t * k);
        if (scores32)
            memcpy(scores32 + (size_t)t * max_slots, sc, sizeof(float) * (size_t)nv);
        free(sc);
    }
}

/* --------------------------------------------------------------- attention */

/*
 * Sparse MLA attention of one query in absorbed (MQA) form [P5 Ch.2; P3
 * forward_mqa / _forward_decode]: h query heads, one shared 576-wide latent
 * key per attended entry, values = the key's first 512 dims.
 *
 * Attended list [P1: SWA indices together with compressed top-k; P4: the
 * selected history concatenated with the recent window]:
 *   SWA entries: positions max(0, p-W+1) .. p, rows swa_rows[pos - swa_base];
 *   compressed entries: idx[0..k) with 0 <= idx < n_slots (others skipped),
 *   each row = e4m3 code * pow2 scale for the 512 nope dims ++ bf16 rope.
 * Entries are not deduplicated.
 *   logit_i = sm_scale * q_h . K_i;  p = softmax(logit);
 *   out_h = sum_i p_i K_i[0:512] (bf16), lse_h = ln sum_i exp(logit_i) (fp32).
 * An empty list gives out = 0 and lse = -inf.
 * Returns 0, or -1 if a window position has no row in swa_rows.
 */
int oracle_sparse_mla(int h, const uint16_t *q, int p, int W, int swa_base,
                      int swa_count, const uint16_t *swa_rows, int n_slots,
                      const uint8_t *codes, const float *scales,
                      const uint16_t *rope, int k, const int32_t *idx,
                      double sm_scale, uint16_t *out, float *lse,
                      double *out64, double *lse64)
{
    int lo = p - W + 1 < 0 ? 0 : p - W + 1;
    int n_swa = W > 0 ? p - lo + 1 : 0;
    int cap = n_swa + (k > 0 ? k : 0);
    double *K = (double *)malloc(sizeof(double) * OR_D * (size_t)(cap > 0 ? cap : 1));
    double *logit = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    int n = 0;

    for (int pos = lo; n_swa > 0 && pos <= p; pos++) {
        if (pos < swa_base || pos >= swa_base + swa_count) {
            free(K);
            free(logit);
            return -1;
        }
        for (int d = 0; d < OR_D; d++)
            K[(size_t)n * OR_D + d] =
                oracle_bf16_value(swa_rows[(size_t)(pos - swa_base) * OR_D + d]);
        n++;
    }
    for (int t = 0; t < k; t++) {
        int s = idx[t];
        if (s < 0 || s >= n_slots)
            continue;
        for (int d = 0; d < OR_DN; d++)
            K[(size_t)n * OR_D + d] = oracle_e4m3_value(codes[(size_t)s * OR_DN + d]) *
                                      (double)scales[(size_t)s * (OR_DN / OR_QB) + d / OR_QB];
        for (int d = 0; d < OR_DR; d++)
            K[(size_t)n * OR_D + OR_DN + d] = oracle_bf16_value(rope[(size_t)s * OR_DR + d]);
        n++;
    }

    for (int hh = 0; hh < h; hh++) {
        double m = -INFINITY, se = 0.0, o[OR_DN];
        const uint16_t *qh = q + (size_t)hh * OR_D;
        for (int i = 0; i < n; i++) {
            double dot = 0.0;
            for (int d = 0; d < OR_D; d++)
                dot += oracle_bf16_value(qh[d]) * K[(size_t)i * OR_D + d];
            logit[i] = sm_scale * dot;
            if (logit[i] > m)
                m = logit[i];
        }
        for (int c = 0; c < OR_DN; c++)
            o[c] = 0.0;
        for (int i = 0; i < n; i++) {
            double e = exp(logit[i] - m);
            se += e;
            for (int c = 0; c < OR_DN; c++)
                o[c] += e * K[(size_t)i * OR_D + c];
        }
        for (int c = 0; c < OR_DN; c++) {
            double v = n > 0 ? o[c] / se : 0.0;
            out[(size_t)hh * OR_DN + c] = oracle_bf16_encode(v);
            if (out64)
                out64[(size_t)hh * OR_DN + c] = v;
        }
        {
            double l = n > 0 ? m + log(se) : -INFINITY;
            lse[hh] = (float)l;
            if (lse64)
                lse64[hh] = l;
        }
    }
    free(K);
    free(logit);
    return 0;
}

/*
 * Batch of n_q queries (decode: one per sequence; prefill: many per
 * sequence).  Per sequence b: SWA rows start at row swa_off[b] of swa_rows
 * and hold positions swa_base[b] .. swa_base[b]+swa_count[b]-1; compressed
 * slots start at row cmp_off[b] of codes/scales/rope, n_slots[b] of them.
 *   q [n_q, h, 576] bf16, idx [n_q, k] (NULL or k == 0: no compressed list)
 *   out [n_q, h, 512] bf16, lse [n_q, h] fp32, out64/lse64 nullable doubles
 * Returns 0, or -1 if any query's window is not covered by its SWA rows.
 */
int oracle_sparse_mla_batch(int n_q, int h, const uint16_t *q,
                            const int32_t *q_pos, const int32_t *q_seq, int W,
                            const int64_t *swa_off, const int32_t *swa_base,
                            const int32_t *swa_count, const uint16_t *swa_rows,
                            const int64_t *cmp_off, const int32_t *n_slots,
                            const uint8_t *codes, const float *scales,
                            const uint16_t *rope, int k, const int32_t *idx,
                            double sm_scale, uint16_t *out, float *lse,
                            double *out64, double *lse64)
{
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int t = 0; t < n_q; t++) {
        int b = q_seq[t];
        int kk = (idx && k > 0) ? k : 0;
        int64_t co = cmp_off ? cmp_off[b] : 0;
        int ns = n_slots ? n_slots[b] : 0;
        int r1 = oracle_sparse_mla(
            h, q + (size_t)t * h * OR_D, q_pos[t], W, swa_base[b], swa_count[b],
            swa_rows + (size_t)swa_off[b] * OR_D, ns,
            codes ? codes + (size_t)co * OR_DN : NULL,
            scales ? scales + (size_t)co * (OR_DN / OR_QB) : NULL,
            rope ? rope + (size_t)co * OR_DR : NULL, kk,
            kk ? idx + (size_t)t * k : NULL, sm_scale,
            out + (size_t)t * h * OR_DN, lse + (size_t)t * h,
            out64 ? out64 + (size_t)t * h * OR_DN : NULL,
            lse64 ? lse64 + (size_t)t * h : NULL);
        if (r1) {
#pragma omp atomic write
            rc = -1;
        }
    }
    return rc;
}

/* Threads an OpenMP region of this library uses (1 without OpenMP). */
int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}

/* ------------------------------------------------ array forms of the codecs */

void oracle_e4m3_decode_array(int64_t n, const uint8_t *in, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e4m3_value(in[i]);
}

void oracle_e4m3_encode_array(int64_t n, const double *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e4m3_encode(in[i]);
}

void oracle_bf16_decode_array(int64_t n, const uint16_t *in, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_value(in[i]);
}

void oracle_bf16_encode_array(int64_t n, const double *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_encode(in[i]);
}

/* The pow2 quantisation scale the compressor picks for a block whose largest
 * magnitude is amax (exposed for the scale-rule pins). */
double oracle_pow2_scale(double amax)
{
    return ldexp(1.0, pow2_exponent_for(amax));
}
