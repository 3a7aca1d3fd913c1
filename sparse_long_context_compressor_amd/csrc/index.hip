// index.hip -- lightning-indexer scores and the per-query global top-k.
//
// Method: "DeepseekV4Attention" (devpress, AMD), Indexer section:
//   I[t][s] = sum_j w[t][j] * ReLU(q[t][j] . k[s]),  H_I heads sharing one
//   key per slot, fp8 keys of 128 dims with one fp32 scale per key;
// "DeepSeek-V4 attention layer types", Indexer / C4A branch: c4a computes a
// global top-k over these scores for every query.
//
// Scores: the contraction [H_I x 128] . [128 x slots] runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).  e4m3 codes convert to bf16 exactly, and the
// bf16 MFMA accumulates at fp32 accuracy; gfx950's fp8 MFMAs accumulate the
// 128 products at a reduced internal precision (measured errors up to 1e-4 of
// sum|p|), which would break exact top-k agreement, so they are not used here.
// The contraction is far below the bf16 ridge (the keys are the traffic), so
// the kernel stays HBM-bound either way.
//
// Top-k: one workgroup per query runs an MSB-first radix select (4 passes of
// 8 bits) over order-preserving 32-bit keys of the fp32 scores, held in LDS,
// then writes the selected slots in increasing slot order; ties at the
// threshold go to the lower slot index.

#include "slc_internal.hpp"

namespace slc {

namespace {

// 16 bytes of e4m3 (4 dwords) at k positions [8s, 8s+8) for s = 0, 1 -> two
// bf16x8 MFMA operands.
__device__ __forceinline__ void e4m3x16_to_operands(u32x4 w, float scale, bf16x8 &s0,
                                                    bf16x8 &s1) {
    u32x2 a = e4m3x4_to_bf16x4(w[0], scale);
    u32x2 b = e4m3x4_to_bf16x4(w[1], scale);
    u32x2 c = e4m3x4_to_bf16x4(w[2], scale);
    u32x2 d = e4m3x4_to_bf16x4(w[3], scale);
    s0 = __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
    s1 = __builtin_bit_cast(bf16x8, u32x4{c[0], c[1], d[0], d[1]});
}

constexpr int kScoreTile = 256;   // slots per workgroup (4 waves x 4 sub-tiles x 16)

}  // namespace

// grid (n_q, ceil(max_slots / 256)), 256 threads.  Lane (g = lane/16, c = lane%16)
// owns index-dim bytes [16g, 16g+16) and [64+16g, 64+16g+16) of its head / key:
// the k-ordering inside the MFMA is the same permutation for both operands, so
// the dot product is unchanged.
template <int HT>
__global__ __launch_bounds__(256) void index_score_kernel(IndexArgs a) {
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int seq = a.q_seq[t];
    int nv = visible_slots(a.q_pos[t], a.ratio, a.n_slots[seq]);
    nv = nv < a.max_slots ? nv : a.max_slots;
    const int s0 = blockIdx.y * kScoreTile;
    if (s0 >= nv) return;

    bf16x8 qa[HT][4];
    float hs[HT][4], hw[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        const uint8_t *qp = a.q + (static_cast<int64_t>(t) * a.h_idx + 16 * ht + c) * kDI;
        u32x4 lo = *reinterpret_cast<const u32x4 *>(qp + 16 * g);
        u32x4 hi = *reinterpret_cast<const u32x4 *>(qp + 64 + 16 * g);
        e4m3x16_to_operands(lo, 1.0f, qa[ht][0], qa[ht][1]);
        e4m3x16_to_operands(hi, 1.0f, qa[ht][2], qa[ht][3]);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int h = 16 * ht + 4 * g + i;
            hs[ht][i] = a.q_scale[static_cast<int64_t>(t) * a.h_idx + h];
            hw[ht][i] = a.w[static_cast<int64_t>(t) * a.h_idx + h];
        }
    }

    // issue all four sub-tiles' key loads first
    u32x4 klo[4], khi[4];
    float ksc[4];
    int64_t krow[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        int s = s0 + 16 * (w + 4 * j) + c;
        krow[j] = s < nv ? pool_row(a.keys, seq, s) : -1;
        if (krow[j] >= 0) {
            const uint8_t *kp = key_code_ptr(a.keys, krow[j]);
            klo[j] = *reinterpret_cast<const u32x4 *>(kp + 16 * g);
            khi[j] = *reinterpret_cast<const u32x4 *>(kp + 64 + 16 * g);
            ksc[j] = *key_scale_ptr(a.keys, krow[j]);
        } else {
            klo[j] = u32x4{0, 0, 0, 0};
            khi[j] = u32x4{0, 0, 0, 0};
            ksc[j] = 0.f;
        }
    }

#pragma unroll
    for (int j = 0; j < 4; j++) {
        int s = s0 + 16 * (w + 4 * j) + c;
        bf16x8 kb[4];
        e4m3x16_to_operands(klo[j], 1.0f, kb[0], kb[1]);
        e4m3x16_to_operands(khi[j], 1.0f, kb[2], kb[3]);
        f32x4 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; st++)
                acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ht][st], kb[st], acc[ht], 0,
                                                                   0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ht++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float v = acc[ht][i] * hs[ht][i] * ksc[j];
                v = v > 0.f ? v : 0.f;
                part += hw[ht][i] * v;
            }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        if (g == 0 && s < nv)
            a.scores[static_cast<int64_t>(t) * a.max_slots + s] = krow[j] >= 0 ? part : -INFINITY;
    }
}

hipError_t launch_index_scores(const IndexArgs &a, hipStream_t stream) {
    dim3 grid(a.n_q, (a.max_slots + kScoreTile - 1) / kScoreTile);
    switch (a.h_idx / 16) {
    case 1: hipLaunchKernelGGL(index_score_kernel<1>, grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(index_score_kernel<2>, grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(index_score_kernel<3>, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(index_score_kernel<4>, grid, dim3(256), 0, stream, a); break;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------- top-k

namespace {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkLdsKeys = 32768;   // 128 KB: scores of up to 32768 visible slots

// Order-preserving map fp32 -> uint32 (larger score -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float s) {
    uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below() {
    return (1ull << (threadIdx.x & 63)) - 1ull;
}

// Block-wide exclusive prefix of per-wave counts; returns this wave's offset
// and writes the block total to *total.  Uses sh[kTopkWaves].
__device__ __forceinline__ int wave_offset(int wave_count, int *sh, int *total) {
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = wave_count;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; i++) {
        int v = sh[i];
        off += i < w ? v : 0;
        tot += v;
    }
    *total = tot;
    __syncthreads();
    return off;
}

}  // namespace

template <bool LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
    __shared__ uint32_t keys_lds[LDS ? kTopkLdsKeys : 1];
    __shared__ uint32_t hist[kTopkWaves][256];
    __shared__ int scan_sh[kTopkWaves];
    __shared__ int sel_sh[2];

    const int t = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6;
    const int seq = a.q_seq[t];
    int n = visible_slots(a.q_pos[t], a.ratio, a.n_slots[seq]);
    n = n < a.max_slots ? n : a.max_slots;
    const int k = a.k;
    const int k_eff = n < k ? n : k;
    int32_t *out = a.idx + static_cast<int64_t>(t) * k;
    const float *sc = a.scores + static_cast<int64_t>(t) * a.max_slots;
    if (tid == 0) a.len[t] = k_eff;

    if (n <= k) {   // everything visible is selected
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }

    if (LDS)
        for (int i = tid; i < n; i += kTopkThreads) keys_lds[i] = order_key(sc[i]);
    auto key_at = [&](int i) -> uint32_t { return LDS ? keys_lds[i] : order_key(sc[i]); };

    // ---- radix select of the k-th largest key ----
    uint32_t prefix = 0;
    int remaining = k;   // how many still to take among keys matching `prefix`
#pragma unroll 1
    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
        for (int i = tid; i < n; i += kTopkThreads) {
            uint32_t kk = key_at(i);
            if ((kk & hi_mask) == prefix) atomicAdd(&hist[w][(kk >> shift) & 255u], 1u);
        }
        __syncthreads();
        // bins from the top: thread b (< 256) owns bin 255 - b
        int cnt = 0;
        if (tid < 256) {
#pragma unroll
            for (int ww = 0; ww < kTopkWaves; ww++) cnt += hist[ww][255 - tid];
        }
        // inclusive scan over tid (bins descending) within waves 0..3
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int v = __shfl_up(incl, o, 64);
            if ((tid & 63) >= o) incl += v;
        }
        if (tid < 256 && (tid & 63) == 63) scan_sh[w] = incl;
        __syncthreads();
        if (tid < 256) {
            int before = 0;
            for (int ww = 0; ww < w; ww++) before += scan_sh[ww];
            int excl = before + incl - cnt;
            if (excl < remaining && excl + cnt >= remaining) {
                sel_sh[0] = 255 - tid;
                sel_sh[1] = remaining - excl;
            }
        }
        __syncthreads();
        prefix |= static_cast<uint32_t>(sel_sh[0]) << shift;
        remaining = sel_sh[1];
        __syncthreads();
    }
    const uint32_t thr = prefix;     // the k-th largest key
    const int take_eq = remaining;   // keys equal to thr to take, lowest slots first

    // ---- ordered write: slots with key > thr, plus the first take_eq with key == thr ----
    int eq_before = 0, sel_before = 0;
    for (int base = 0; base < n; base += kTopkThreads) {
        int i = base + tid;
        uint32_t kk = i < n ? key_at(i) : 0u;
        bool gt = i < n && kk > thr;
        bool eq = i < n && kk == thr;
        uint64_t beq = __ballot(eq);
        int eq_tot;
        int eq_off = wave_offset(__popcll(beq), scan_sh, &eq_tot);
        int eq_rank = eq_before + eq_off + __popcll(beq & lanes_below());
        bool sel = gt || (eq && eq_rank < take_eq);
        uint64_t bsel = __ballot(sel);
        int sel_tot;
        int sel_off = wave_offset(__popcll(bsel), scan_sh, &sel_tot);
        if (sel) out[sel_before + sel_off + __popcll(bsel & lanes_below())] = i;
        eq_before += eq_tot;
        sel_before += sel_tot;
    }
    for (int i = k_eff + tid; i < k; i += kTopkThreads) out[i] = -1;
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
    if (a.max_slots <= kTopkLdsKeys)
        hipLaunchKernelGGL(topk_kernel<true>, dim3(a.n_q), dim3(kTopkThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(topk_kernel<false>, dim3(a.n_q), dim3(kTopkThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace slc
