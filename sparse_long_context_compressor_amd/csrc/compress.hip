// compress.hip -- fused compressor kernel: window pooling -> RMSNorm -> RoPE ->
// FP8 quantisation -> paged store, one slot per wave (r = 4) or per workgroup
// (r = 128); and the SWA KV insert (RoPE -> FP8 quantisation -> paged store of
// single tokens into an fp8 sliding-window pool), which shares the row format.
//
// Method: "DeepseekV4Attention" (devpress, AMD), DeepseekCompressor forward
// and the CSA/HCA compressor sections (softmax-gated pooling of the window's
// kv by per-channel scores; RMSNorm; GPT-J RoPE on the last 64 dims at
// position (pos // r) * r; fp8 nope + bf16 rope with one scale per 64 dims);
// "From MLA to CSA + HCA" 5.1 (slot j of r = 4 covers [4j-4, 4j+3]), 5.2
// (r = 128 covers [128j, 128j+127]), 6.2 (one fused kernel: intermediates stay
// in registers), 6.3 (slot j -> block j / 64, row j % 64).
//
// Layout on the wave: lane l owns nope channels [8l, 8l+8) and rope channel
// 512 + l.  A quantisation block (64 channels) is then 8 adjacent lanes, the
// RoPE pair (512+2i, 513+2i) is the lane pair (2i, 2i+1), and every token row
// is read with fully coalesced 16/32-byte loads.

#include "slc_internal.hpp"

namespace slc {

namespace {

struct PoolState {
    float m[9], l[9], acc[9];   // running max, sum of exp, weighted kv (8 nope + 1 rope)
};

__device__ __forceinline__ void state_init(PoolState &s) {
#pragma unroll
    for (int i = 0; i < 9; i++) {
        s.m[i] = -INFINITY;
        s.l[i] = 0.f;
        s.acc[i] = 0.f;
    }
}

__device__ __forceinline__ void state_add(PoolState &s, int i, float sc, float x) {
    float mn = fmaxf(s.m[i], sc);
    float a = __expf(s.m[i] - mn);   // 0 when m was -inf
    float e = __expf(sc - mn);
    s.l[i] = s.l[i] * a + e;
    s.acc[i] = s.acc[i] * a + e * x;
    s.m[i] = mn;
}

// Fold token t's kv/score row into the lane's 9 channels.
__device__ __forceinline__ void pool_token(PoolState &s, const uint16_t *kv, const float *score,
                                           int64_t t, int lane) {
    const uint16_t *kr = kv + t * kD;
    const float *sr = score + t * kD;
    u32x4 kw = *reinterpret_cast<const u32x4 *>(kr + 8 * lane);
    f32x4 s0 = *reinterpret_cast<const f32x4 *>(sr + 8 * lane);
    f32x4 s1 = *reinterpret_cast<const f32x4 *>(sr + 8 * lane + 4);
    uint16_t kr_rope = kr[kDN + lane];
    float s_rope = sr[kDN + lane];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        state_add(s, 2 * i, i < 2 ? s0[2 * i] : s1[2 * i - 4], __uint_as_float(kw[i] << 16));
        state_add(s, 2 * i + 1, i < 2 ? s0[2 * i + 1] : s1[2 * i - 3],
                  __uint_as_float(kw[i] & 0xffff0000u));
    }
    state_add(s, 8, s_rope, bf16_to_f32(kr_rope));
}

// Smallest e with amax <= 448 * 2^e (exact comparisons), at least -126; 0 for
// amax == 0.
__device__ __forceinline__ int pow2_exponent(float amax) {
    if (!(amax > 0.f)) return 0;
    int ex;
    frexpf(amax, &ex);            // amax = f * 2^ex, f in [0.5, 1); 448 = 0.875 * 2^9
    int e = ex - 9;
    while (amax > ldexpf(448.f, e)) e++;
    while (amax <= ldexpf(448.f, e - 1)) e--;
    // the scale is stored as an fp32 power of two, normal down to 2^-126:
    // tinier blocks share that scale (their codes round toward zero)
    return e < -126 ? -126 : e;
}

// GPT-J RoPE of the lane's rope channel at position pos: the pair
// (512+2i, 513+2i) is the lane pair (2i, 2i+1).
__device__ __forceinline__ float rope_lane(float v, int lane, int pos, const float *cos_sin) {
    float other = __shfl_xor(v, 1, 64);
    int pi = lane >> 1;
    float c = cos_sin[static_cast<int64_t>(pos) * kDR + pi];
    float s = cos_sin[static_cast<int64_t>(pos) * kDR + kDR / 2 + pi];
    return (lane & 1) ? (other * s + v * c) : (v * c - other * s);
}

__device__ __forceinline__ void store_prequant(float *pq, const float (&y)[9], int lane) {
    *reinterpret_cast<f32x4 *>(pq + 8 * lane) = f32x4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4 *>(pq + 8 * lane + 4) = f32x4{y[4], y[5], y[6], y[7]};
    pq[kDN + lane] = y[8];
}

// The wave's row y in the cache row format, stored at physical row `row` of a
// pool with the compressed-row layout: per 64-dim block (lanes 8b .. 8b+7)
// the pow2 scale of its amax and e4m3 codes of y / scale; rope -> bf16.
__device__ __forceinline__ void quant_store(const float (&y)[9], int lane, slc_pool_t pool,
                                            int64_t row) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(y[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    int e = pow2_exponent(amax);
    float inv_scale = ldexpf(1.f, -e);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        w0 |= f32_to_e4m3(y[i] * inv_scale) << (8 * i);
        w1 |= f32_to_e4m3(y[4 + i] * inv_scale) << (8 * i);
    }
    uint8_t *dst = cmp_row_ptr(pool, row);
    *reinterpret_cast<u32x2 *>(dst + 8 * lane) = u32x2{w0, w1};
    reinterpret_cast<uint16_t *>(dst + kDN)[lane] = f32_to_bf16(y[8]);
    if ((lane & 7) == 0) cmp_scale_ptr(pool, row)[lane >> 3] = ldexpf(1.f, e);
}

// Smallest e with amax <= 6 * 2^e (e2m1's largest magnitude), at least -127;
// 0 for amax == 0.
__device__ __forceinline__ int pow2_exponent_e2m1(float amax) {
    if (!(amax > 0.f)) return 0;
    int ex;
    frexpf(amax, &ex);            // amax = f * 2^ex, f in [0.5, 1); 6 = 0.75 * 2^3
    int e = ex - 3;
    while (amax > ldexpf(6.f, e)) e++;
    while (amax <= ldexpf(6.f, e - 1)) e--;
    return e < -127 ? -127 : e;   // E8M0's smallest scale (byte 0 = 2^-127)
}

// Nearest e2m1 code of x (|x| <= 6 by the caller's scale), ties to the even
// code: the thresholds are the midpoints between adjacent magnitudes 0, 0.5,
// 1, 1.5, 2, 3, 4, 6, taken with > where the lower code is even.
__device__ __forceinline__ uint32_t e2m1_code(float x) {
    const float m = fabsf(x);
    const uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
                       (m >= 3.5f) + (m > 5.f);
    return c | (x < 0.f ? 8u : 0u);
}

// RMSNorm, RoPE, quantise and store one pooled slot held by one wave.
// prequant rows: at the slot's physical row (pq_index < 0) or at pq_index.
__device__ __forceinline__ void finish_slot(const float (&pooled)[9], int lane, int seq, int slot,
                                            int ratio, const float *gamma, float eps,
                                            const float *cos_sin, int max_pos, slc_pool_t pool,
                                            float *prequant, int64_t pq_index = -1) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 9; i++) ss += pooled[i] * pooled[i];
    ss = wave_sum(ss);
    float inv = 1.0f / sqrtf(ss * (1.0f / kD) + eps);

    float y[9];
    f32x4 g0 = *reinterpret_cast<const f32x4 *>(gamma + 8 * lane);
    f32x4 g1 = *reinterpret_cast<const f32x4 *>(gamma + 8 * lane + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        y[i] = pooled[i] * inv * g0[i];
        y[4 + i] = pooled[4 + i] * inv * g1[i];
    }
    y[8] = pooled[8] * inv * gamma[kDN + lane];

    int pos = ratio * slot;
    if (pos >= max_pos) return;   // anchor outside the table: slot not written
    y[8] = rope_lane(y[8], lane, pos, cos_sin);

    int64_t row = pool_row(pool, seq, slot);
    if (row < 0) return;
    if (prequant) store_prequant(prequant + (pq_index < 0 ? row : pq_index) * kD, y, lane);
    quant_store(y, lane, pool, row);
}

// Streaming state rows: entry of (seq, pos) in a pool of `rows` rows per
// block, each 2 * width floats (kv blocks, then score blocks); null if absent.
__device__ __forceinline__ float *state_row(const slc_pool_t &p, int rows, int width, int seq,
                                            int pos) {
    if (pos < 0) return nullptr;
    const int lb = pos / rows;
    if (lb >= p.table_stride) return nullptr;
    const int32_t pb = p.block_table[static_cast<int64_t>(seq) * p.table_stride + lb];
    if (pb < 0 || pb >= p.n_blocks) return nullptr;
    return reinterpret_cast<float *>(p.base) +
           (static_cast<int64_t>(pb) * rows + pos % rows) * (2 * width);
}

// Fold one state entry's block `blk` into the lane's 9 channels (logits are
// stored with the bias already added).
__device__ __forceinline__ void pool_state(PoolState &s, const float *row, int width, int blk,
                                           int lane) {
    const float *kv = row + blk * kD, *sc = row + width + blk * kD;
    const f32x4 k0 = *reinterpret_cast<const f32x4 *>(kv + 8 * lane);
    const f32x4 k1 = *reinterpret_cast<const f32x4 *>(kv + 8 * lane + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sc + 8 * lane);
    const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sc + 8 * lane + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        state_add(s, i, s0[i], k0[i]);
        state_add(s, 4 + i, s1[i], k1[i]);
    }
    state_add(s, 8, sc[kDN + lane], kv[kDN + lane]);
}

}  // namespace

// r = 4: one wave per slot, 4 slots per workgroup; window = [4j-4, 4j+3] ∩ [0, L).
__global__ __launch_bounds__(256) void compress_r4_kernel(CompressArgs a) {
    const int lane = threadIdx.x & 63;
    const int seq = blockIdx.y;
    const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
    int64_t t0 = a.cu_seqlens[seq];
    int L = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    L = L < a.max_seqlen ? L : a.max_seqlen;
    const int n_slots = (L + 3) / 4;
    if (L <= 0 || slot >= n_slots) return;

    int lo = 4 * slot - 4, hi = 4 * slot + 3;
    lo = lo < 0 ? 0 : lo;
    hi = hi > L - 1 ? L - 1 : hi;
    PoolState st;
    state_init(st);
    for (int t = lo; t <= hi; t++) pool_token(st, a.kv, a.score, t0 + t, lane);
    float pooled[9];
#pragma unroll
    for (int i = 0; i < 9; i++) pooled[i] = st.acc[i] / st.l[i];
    finish_slot(pooled, lane, seq, slot, 4, a.gamma, a.eps, a.cos_sin, a.max_pos, a.pool,
                a.prequant);
}

// r = 128: one workgroup per slot; 4 waves pool 32 tokens each, wave 0 merges.
__global__ __launch_bounds__(256) void compress_r128_kernel(CompressArgs a) {
    __shared__ float part_m[4][kD], part_l[4][kD], part_acc[4][kD];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int seq = blockIdx.y;
    const int slot = blockIdx.x;
    int64_t t0 = a.cu_seqlens[seq];
    int L = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    L = L < a.max_seqlen ? L : a.max_seqlen;
    const int n_slots = (L + 127) / 128;
    if (L <= 0 || slot >= n_slots) return;

    int lo = 128 * slot + 32 * w, hi = lo + 31;
    hi = hi > L - 1 ? L - 1 : hi;
    PoolState st;
    state_init(st);
    for (int t = lo; t <= hi; t++) pool_token(st, a.kv, a.score, t0 + t, lane);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        part_m[w][8 * lane + i] = st.m[i];
        part_l[w][8 * lane + i] = st.l[i];
        part_acc[w][8 * lane + i] = st.acc[i];
    }
    part_m[w][kDN + lane] = st.m[8];
    part_l[w][kDN + lane] = st.l[8];
    part_acc[w][kDN + lane] = st.acc[8];
    __syncthreads();
    if (w != 0) return;

    float pooled[9];
#pragma unroll
    for (int i = 0; i < 9; i++) {
        int d = i < 8 ? 8 * lane + i : kDN + lane;
        float m = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) m = fmaxf(m, part_m[ww][d]);
        float l = 0.f, acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) {
            float sc = part_l[ww][d] > 0.f ? __expf(part_m[ww][d] - m) : 0.f;
            l += part_l[ww][d] * sc;
            acc += part_acc[ww][d] * sc;
        }
        pooled[i] = acc / l;
    }
    finish_slot(pooled, lane, seq, slot, 128, a.gamma, a.eps, a.cos_sin, a.max_pos, a.pool,
                a.prequant);
}

// SWA KV insert, one token per wave: RoPE at the token's own position, then
// the cache row format, written at the position's row of its sequence.
// "From MLA to CSA + HCA" 6.2 (the fused KV insert: GPT-J RoPE, fp8
// quantisation, paged write) and 5.5 (the SWA cache's fp8 row).
__device__ __forceinline__ void swa_insert_token(const SwaInsertArgs &a, int t, int lane) {
    const int seq = a.tok_seq[t], pos = a.tok_pos[t];
    if (pos < 0 || pos >= a.max_pos) return;        // uniform over the wave
    const uint16_t *kr = a.kv + static_cast<int64_t>(t) * kD;
    const u32x4 kw = *reinterpret_cast<const u32x4 *>(kr + 8 * lane);
    float y[9];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        y[2 * i] = __uint_as_float(kw[i] << 16);
        y[2 * i + 1] = __uint_as_float(kw[i] & 0xffff0000u);
    }
    y[8] = rope_lane(bf16_to_f32(kr[kDN + lane]), lane, pos, a.cos_sin);
    if (a.prequant) store_prequant(a.prequant + static_cast<int64_t>(t) * kD, y, lane);
    const int64_t row = pool_row(a.pool, seq, pos);
    if (row < 0) return;
    quant_store(y, lane, a.pool, row);
}

__global__ __launch_bounds__(256) void swa_insert_kernel(SwaInsertArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.n_tok) return;
    swa_insert_token(a, t, lane);
}

hipError_t launch_swa_insert(const SwaInsertArgs &a, hipStream_t stream) {
    if (a.n_tok <= 0) return hipSuccess;
    hipLaunchKernelGGL(swa_insert_kernel, dim3((a.n_tok + 3) / 4), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// Streaming compressor, step 1 ("DeepseekV4Attention", save_partial_states):
// each token's kv blocks (as fp32) and score blocks plus the APE row
// pos % ratio go to its state row.  One workgroup per token.
__global__ __launch_bounds__(256) void stream_save_kernel(StreamArgs a) {
    const int t = blockIdx.x;
    const int width = (a.ratio == 4 ? 2 : 1) * a.dim;
    const int pos = a.tok_pos[t];
    float *row = state_row(a.state, a.state_block, width, a.tok_seq[t], pos);
    if (!row) return;
    const uint16_t *kv = a.kv + static_cast<int64_t>(t) * width;
    const float *sc = a.score + static_cast<int64_t>(t) * width;
    const float *ape = a.ape + static_cast<int64_t>(pos % a.ratio) * width;
    for (int c = threadIdx.x; c < width; c += 256) {
        row[c] = bf16_to_f32(kv[c]);
        row[width + c] = sc[c] + ape[c];
    }
}

// Step 2 (the fused compress -> RMSNorm -> RoPE -> quantise -> store): a
// token at position r*j + r - 1 emits slot j from the state rows of its
// window.  r = 4: one wave per token (four per workgroup); entries are the
// block-0 halves of tokens 4j-4 .. 4j-1 and the block-1 halves of 4j ..
// 4j+3 ("DeepseekV4Attention", CSA compressor: the older group brings C_a,
// the newer C_b).  r = 128: one workgroup per token, four waves pooling 32
// entries each, merged through LDS.  Absent state rows are skipped.
// own: the emitting token's own state row (in LDS) when the caller has it,
// else null (read from the state pool like the others).
__device__ __forceinline__ void emit_r4(const StreamArgs &a, int t, int seq, int pos,
                                        const float *own, int lane) {
    const int slot = pos / 4;
    PoolState st;
    state_init(st);
    for (int e = 0; e < 8; e++) {
        const int p = 4 * slot - 4 + e;
        const float *row = (own && p == pos) ? own : state_row(a.state, a.state_block, 2 * kD, seq, p);
        if (row) pool_state(st, row, 2 * kD, e < 4 ? 0 : 1, lane);
    }
    float pooled[9];
#pragma unroll
    for (int i = 0; i < 9; i++) pooled[i] = st.l[i] > 0.f ? st.acc[i] / st.l[i] : 0.f;
    finish_slot(pooled, lane, seq, slot, 4, a.gamma, a.eps, a.cos_sin, a.max_pos, a.pool,
                a.prequant, t);
}

__global__ __launch_bounds__(256) void stream_emit_r4_kernel(StreamArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.n_tok) return;
    const int pos = a.tok_pos[t], seq = a.tok_seq[t];
    if (pos < 0 || (pos + 1) % 4 != 0) return;           // uniform over the wave
    emit_r4(a, t, seq, pos, nullptr, lane);
}

// r = 128: the workgroup's four waves pool 32 positions each, merged in LDS.
__device__ __forceinline__ void emit_r128(const StreamArgs &a, int t, int seq, int pos,
                                          const float *own, int lane, int w,
                                          float (*part_m)[kD], float (*part_l)[kD],
                                          float (*part_acc)[kD]) {
    const int slot = pos / 128;
    PoolState st;
    state_init(st);
    for (int e = 32 * w; e < 32 * w + 32; e++) {
        const int p = 128 * slot + e;
        const float *row = (own && p == pos) ? own : state_row(a.state, a.state_block, kD, seq, p);
        if (row) pool_state(st, row, kD, 0, lane);
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
        part_m[w][8 * lane + i] = st.m[i];
        part_l[w][8 * lane + i] = st.l[i];
        part_acc[w][8 * lane + i] = st.acc[i];
    }
    part_m[w][kDN + lane] = st.m[8];
    part_l[w][kDN + lane] = st.l[8];
    part_acc[w][kDN + lane] = st.acc[8];
    __syncthreads();
    if (w != 0) return;
    float pooled[9];
#pragma unroll
    for (int i = 0; i < 9; i++) {
        const int d = i < 8 ? 8 * lane + i : kDN + lane;
        float m = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) m = fmaxf(m, part_m[ww][d]);
        float l = 0.f, acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) {
            const float sc = part_l[ww][d] > 0.f ? __expf(part_m[ww][d] - m) : 0.f;
            l += part_l[ww][d] * sc;
            acc += part_acc[ww][d] * sc;
        }
        pooled[i] = l > 0.f ? acc / l : 0.f;
    }
    finish_slot(pooled, lane, seq, slot, 128, a.gamma, a.eps, a.cos_sin, a.max_pos, a.pool,
                a.prequant, t);
}

__global__ __launch_bounds__(256) void stream_emit_r128_kernel(StreamArgs a) {
    __shared__ float part_m[4][kD], part_l[4][kD], part_acc[4][kD];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = blockIdx.x;
    const int pos = a.tok_pos[t], seq = a.tok_seq[t];
    if (pos < 0 || (pos + 1) % 128 != 0) return;          // uniform over the workgroup
    emit_r128(a, t, seq, pos, nullptr, lane, w, part_m, part_l, part_acc);
}

// The indexer's key compressor (dim 128, ratio 4): one wave per token; lane
// l holds dims 2l, 2l+1, so the RoPE pair (64+2i, 65+2i) is lane 32+i's own
// two dims.  Pool as the latent r = 4 emit, RMSNorm over 128 dims, RoPE at
// 4j, one pow2 scale for the key, e4m3 codes into the KEY pool.
__device__ __forceinline__ void emit_keys(const StreamArgs &a, int t, int seq, int pos,
                                          const float *own, int lane) {
    const int slot = pos / 4;
    constexpr int kW = 2 * kDI;                          // floats per half state row
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f}, acc[2] = {0.f, 0.f};
    for (int e = 0; e < 8; e++) {
        const int p = 4 * slot - 4 + e;
        const float *row = (own && p == pos) ? own : state_row(a.state, a.state_block, kW, seq, p);
        if (!row) continue;
        const int blk = e < 4 ? 0 : 1;
        const f32x2 kv = *reinterpret_cast<const f32x2 *>(row + blk * kDI + 2 * lane);
        const f32x2 sc = *reinterpret_cast<const f32x2 *>(row + kW + blk * kDI + 2 * lane);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const float mn = fmaxf(m[i], sc[i]);
            const float al = __expf(m[i] - mn), ex = __expf(sc[i] - mn);
            l[i] = l[i] * al + ex;
            acc[i] = acc[i] * al + ex * kv[i];
            m[i] = mn;
        }
    }
    float y[2];
#pragma unroll
    for (int i = 0; i < 2; i++) y[i] = l[i] > 0.f ? acc[i] / l[i] : 0.f;
    const float ss = wave_sum(y[0] * y[0] + y[1] * y[1]);
    const float inv = 1.0f / sqrtf(ss * (1.0f / kDI) + a.eps);
    const f32x2 gm = *reinterpret_cast<const f32x2 *>(a.gamma + 2 * lane);
    y[0] = y[0] * inv * gm[0];
    y[1] = y[1] * inv * gm[1];
    const int anchor = 4 * slot;
    if (anchor >= a.max_pos) return;
    if (lane >= 32) {
        const int i = lane - 32;
        const float c = a.cos_sin[static_cast<int64_t>(anchor) * kDR + i];
        const float s = a.cos_sin[static_cast<int64_t>(anchor) * kDR + kDR / 2 + i];
        const float y0 = y[0], y1 = y[1];
        y[0] = y0 * c - y1 * s;
        y[1] = y0 * s + y1 * c;
    }
    const int64_t row = pool_row(a.pool, seq, slot);
    if (row < 0) return;
    if (a.prequant)
        *reinterpret_cast<f32x2 *>(a.prequant + static_cast<int64_t>(t) * kDI + 2 * lane) = f32x2{y[0], y[1]};
    if (a.key_fp4) {
        // MXFP4: block b = lanes 16b .. 16b+15 (dims 32b .. 32b+31); byte l of
        // the key holds dims 2l (low nibble) and 2l+1
        float bmax = fmaxf(fabsf(y[0]), fabsf(y[1]));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 1, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 2, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 4, 64));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 8, 64));
        const int e = pow2_exponent_e2m1(bmax);
        const float inv_scale = ldexpf(1.f, -e);
        const uint32_t byte = e2m1_code(y[0] * inv_scale) | (e2m1_code(y[1] * inv_scale) << 4);
        uint8_t *base = reinterpret_cast<uint8_t *>(a.pool.base) + (row / kBR) * SLC_KEY4_BLOCK_BYTES;
        base[(row % kBR) * (kDI / 2) + lane] = static_cast<uint8_t>(byte);
        if ((lane & 15) == 0)
            base[SLC_KEY4_SCALE_OFFSET + (row % kBR) * 4 + (lane >> 4)] = static_cast<uint8_t>(e + 127);
        return;
    }
    const float amax = wave_max(fmaxf(fabsf(y[0]), fabsf(y[1])));
    const int e = pow2_exponent(amax);
    const float inv_scale = ldexpf(1.f, -e);
    const uint32_t code = f32_to_e4m3(y[0] * inv_scale) | (f32_to_e4m3(y[1] * inv_scale) << 8);
    uint8_t *base = reinterpret_cast<uint8_t *>(a.pool.base) + (row / kBR) * SLC_KEY_BLOCK_BYTES;
    reinterpret_cast<uint16_t *>(base + (row % kBR) * kDI)[lane] = static_cast<uint16_t>(code);
    if (lane == 0)
        reinterpret_cast<float *>(base + SLC_KEY_SCALE_OFFSET)[row % kBR] = ldexpf(1.f, e);
}

__global__ __launch_bounds__(256) void stream_emit_keys_kernel(StreamArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.n_tok) return;
    const int pos = a.tok_pos[t], seq = a.tok_seq[t];
    if (pos < 0 || (pos + 1) % 4 != 0) return;           // uniform over the wave
    emit_keys(a, t, seq, pos, nullptr, lane);
}

// Both steps in one launch, for calls that bring at most one token per
// sequence (a decode step): the window's other positions were saved by
// earlier calls, and the token's own row is pooled from LDS.  One workgroup
// per token.
struct StepLds {
    float own[4 * kD];
    float part_m[4][kD], part_l[4][kD], part_acc[4][kD];
};

__device__ __forceinline__ void stream_step(const StreamArgs &a, int t, StepLds &lds) {
    float *own = lds.own;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int pos = a.tok_pos[t], seq = a.tok_seq[t];
    if (pos < 0) return;                                  // uniform over the workgroup
    const int width = (a.ratio == 4 ? 2 : 1) * a.dim;
    float *row = state_row(a.state, a.state_block, width, seq, pos);
    const uint16_t *kv = a.kv + static_cast<int64_t>(t) * width;
    const float *sc = a.score + static_cast<int64_t>(t) * width;
    const float *ape = a.ape + static_cast<int64_t>(pos % a.ratio) * width;
    for (int c = threadIdx.x; c < width; c += 256) {
        const float k = bf16_to_f32(kv[c]), v = sc[c] + ape[c];
        own[c] = k;
        own[width + c] = v;
        if (row) {
            row[c] = k;
            row[width + c] = v;
        }
    }
    __syncthreads();
    if ((pos + 1) % a.ratio != 0) return;
    const float *mine = row ? own : nullptr;              // an unmapped row is skipped, as in the pool
    if (a.dim == kDI) {
        if (w == 0) emit_keys(a, t, seq, pos, mine, lane);
    } else if (a.ratio == 4) {
        if (w == 0) emit_r4(a, t, seq, pos, mine, lane);
    } else {
        emit_r128(a, t, seq, pos, mine, lane, w, lds.part_m, lds.part_l, lds.part_acc);
    }
}

__global__ __launch_bounds__(256) void stream_step_kernel(StreamArgs a) {
    __shared__ __attribute__((aligned(16))) StepLds lds;
    stream_step(a, blockIdx.x, lds);
}

// A decode step's per-token writers in one launch: workgroups [0, nl) run
// the latent compressor's step for token b, [nl, nl + nk) the index-key
// compressor's, and the rest insert the tokens' SWA rows, four per
// workgroup.  The three write disjoint pools.
__global__ __launch_bounds__(256) void step_writers_kernel(StreamArgs lat, StreamArgs keys,
                                                           SwaInsertArgs swa, int nl, int nk) {
    __shared__ __attribute__((aligned(16))) StepLds lds;
    const int b = blockIdx.x;
    if (b < nl) {
        stream_step(lat, b, lds);
    } else if (b < nl + nk) {
        stream_step(keys, b - nl, lds);
    } else {
        const int t = (b - nl - nk) * 4 + (threadIdx.x >> 6);
        if (t < swa.n_tok) swa_insert_token(swa, t, threadIdx.x & 63);
    }
}

hipError_t launch_step_writers(const StreamArgs *lat, const StreamArgs *keys,
                               const SwaInsertArgs *swa, hipStream_t stream) {
    const int nl = lat ? lat->n_tok : 0, nk = keys ? keys->n_tok : 0;
    const int ns = swa ? (swa->n_tok + 3) / 4 : 0;
    if (nl + nk + ns == 0) return hipSuccess;
    const StreamArgs none{};
    const SwaInsertArgs no_swa{};
    hipLaunchKernelGGL(step_writers_kernel, dim3(nl + nk + ns), dim3(256), 0, stream,
                       lat ? *lat : none, keys ? *keys : none, swa ? *swa : no_swa, nl, nk);
    return hipGetLastError();
}

hipError_t launch_compress_stream(const StreamArgs &a, bool one_per_seq, hipStream_t stream) {
    if (a.n_tok <= 0) return hipSuccess;
    if (one_per_seq) {
        hipLaunchKernelGGL(stream_step_kernel, dim3(a.n_tok), dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(stream_save_kernel, dim3(a.n_tok), dim3(256), 0, stream, a);
    if (a.dim == kDI)
        hipLaunchKernelGGL(stream_emit_keys_kernel, dim3((a.n_tok + 3) / 4), dim3(256), 0, stream, a);
    else if (a.ratio == 4)
        hipLaunchKernelGGL(stream_emit_r4_kernel, dim3((a.n_tok + 3) / 4), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(stream_emit_r128_kernel, dim3(a.n_tok), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs &a, int n_seq, hipStream_t stream) {
    if (a.ratio == 4) {
        int max_slots = (a.max_seqlen + 3) / 4;
        dim3 grid((max_slots + 3) / 4, n_seq);
        hipLaunchKernelGGL(compress_r4_kernel, grid, dim3(256), 0, stream, a);
    } else {
        int max_slots = (a.max_seqlen + 127) / 128;
        dim3 grid(max_slots, n_seq);
        hipLaunchKernelGGL(compress_r128_kernel, grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace slc
