// topk.hip -- per-query global top-k over the lightning-indexer scores.
//
// Method: "DeepSeek-V4 attention layer types", Indexer / C4A branch: c4a
// computes a global top-k over the indexer scores for every query (the
// IndexCache freq2 page: lists shorter than k are filled with -1).
//
// One workgroup of 1024 threads per query.  The select itself (select.hpp)
// is a radix search over order-preserving 32-bit keys: one histogram of 2048
// equal bins over [min key, max key] finds the bin holding the k-th largest
// key, its few candidates are ranked exactly (key descending, slot
// ascending), and one ordered write places every selected slot in increasing
// slot order, ties at the threshold going to the lower slot.  A prefilter by
// group maxima first cuts the list to a few per cent of it.

#include "slc_internal.hpp"
#include "select.hpp"

namespace slc {

// ------------------------------------------------------------------- top-k

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Block-wide exclusive scan of two counts (sh: 2 * kTopkWaves ints).
__device__ __forceinline__ void block_scan2(int a, int b, int *sh, int &a_before, int &b_before) {
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    if (lane == 63) {
        sh[w] = ia;
        sh[kTopkWaves + w] = ib;
    }
    __syncthreads();
    // fixed trip count: every read is issued at once (a loop to w would wait
    // on each in turn)
    int pa = 0, pb = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; i++) {
        pa += i < w ? sh[i] : 0;
        pb += i < w ? sh[kTopkWaves + i] : 0;
    }
    a_before = pa + ia - a;
    b_before = pb + ib - b;
}

}  // namespace

// L2 warm-up for the attention that follows the select (blocks past the
// queries' when the launcher adds them): reads, and discards, query t's
// inputs that do not depend on the selection -- its query heads and the
// latent rows of its window -- so that the decode finds them in the L2 of
// this XCD (block t' = t + 8m shares blockIdx % 8 with the decode's blocks of
// query t).  Every load is in bounds: rows of absent blocks read the query
// instead.  blk: scratch LDS for up to 32 block ids.
// F8: the SWA pool has the compressed-row layout (640 bytes of codes and rope
// per row, then 32 bytes of scales in the block's scale area).
template <int THREADS, bool F8>
__device__ __forceinline__ void warm_attention_inputs(const TopkArgs &a, int t, int32_t *blk) {
    const int tid = threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    constexpr int kQUnits = kD * 2 / 16;                // 16-byte units per bf16 latent row (72)
    constexpr int kRowUnits = F8 ? (SLC_CMP_ROW_BYTES + 32) / 16 : kQUnits;   // per pool row
    const u32x4 *qp = reinterpret_cast<const u32x4 *>(a.warm_q + static_cast<int64_t>(t) * a.warm_heads * kD);
    const int qunits = a.warm_heads * kQUnits;
    for (int u0 = 0; u0 < qunits; u0 += 4 * THREADS) {
        u32x4 v[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int u = u0 + THREADS * i + tid;
            v[i] = qp[u < qunits ? u : 0];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) acc ^= v[i];
    }
    const slc_pool_t &sp = a.warm_swa;
    const int seq = a.q_seq[t], p = a.q_pos[t];
    const int lo = p - a.warm_window + 1 > 0 ? p - a.warm_window + 1 : 0;
    const int rows = p - lo + 1;
    if (sp.base && a.warm_window > 0 && rows > 0) {
        const int lb0 = lo >> 6, nb = (p >> 6) - lb0 + 1;   // at most 17 blocks (window <= 1024)
        if (tid < nb && tid < 32) {
            const int64_t lb = lb0 + tid;
            const int32_t pb = lb < sp.table_stride ? sp.block_table[static_cast<int64_t>(seq) * sp.table_stride + lb] : -1;
            blk[tid] = pb >= 0 && pb < sp.n_blocks ? pb : -1;
        }
        __syncthreads();
        const int total = rows * kRowUnits;
        const uint8_t *base = reinterpret_cast<const uint8_t *>(sp.base);
        for (int u0 = 0; u0 < total; u0 += 4 * THREADS) {
            u32x4 v[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int u = u0 + THREADS * i + tid;
                const int uu = u < total ? u : 0;
                const int r = lo + uu / kRowUnits, j = uu % kRowUnits;
                const int32_t pb = blk[(r >> 6) - lb0];
                const uint8_t *src;
                if (F8)
                    src = base + static_cast<int64_t>(pb) * SLC_CMP_BLOCK_BYTES +
                          (j < SLC_CMP_ROW_BYTES / 16
                               ? (r & (kBR - 1)) * SLC_CMP_ROW_BYTES + 16 * j
                               : SLC_CMP_SCALE_OFFSET + (r & (kBR - 1)) * 32 + 16 * (j - SLC_CMP_ROW_BYTES / 16));
                else
                    src = base + (static_cast<int64_t>(pb) * kBR + (r & (kBR - 1))) * (kD * 2) + 16 * j;
                v[i] = *(pb >= 0 ? reinterpret_cast<const u32x4 *>(src) : qp);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) acc ^= v[i];
        }
    }
    __asm__ volatile("" ::"v"(acc[0]), "v"(acc[1]), "v"(acc[2]), "v"(acc[3]));   // keeps the loads
}

// One 1024-thread workgroup per query, R scores per thread (R >= 4): wave w
// owns slots [64Rw, 64R(w+1)) and lane l reads slots 64Rw + 256q + 4l + e
// (e < 4) with one 16-byte load per round q, so the wave's slots run in
// (q, lane, e) order; select_row (select.hpp) prefilters by group maxima and
// selects.  1024 threads: with 256 (one wave per SIMD) the phases' latencies
// were exposed (14.4 us on the 64K decode against 10.0), 512 measured no
// better.
constexpr int kCandCap = 4096;

template <int THREADS, int R>
__global__ __launch_bounds__(THREADS) void topk_kernel(TopkArgs a) {
    static_assert(R >= 4, "16-byte score loads");
    constexpr int R4 = R / 4, WAVES = THREADS / 64;
    __shared__ __attribute__((aligned(16))) uint32_t hist[hist_words<THREADS>()];    // 16 KB
    __shared__ __attribute__((aligned(16))) uint32_t cand_key[kCandCap];             // 16 KB
    __shared__ int32_t cand_slot[kCandCap];                                          // 16 KB
    __shared__ int red[3 * WAVES];
    __shared__ int sh[8];

    if (static_cast<int>(blockIdx.x) >= a.n_q) {       // L2 warm-up blocks (and padding)
        const int t = static_cast<int>(blockIdx.x) - ((a.n_q + 7) & ~7);
        if (t >= 0 && t < a.n_q) {
            if (a.warm_swa_fp8) warm_attention_inputs<THREADS, true>(a, t, reinterpret_cast<int32_t *>(hist));
            else warm_attention_inputs<THREADS, false>(a, t, reinterpret_cast<int32_t *>(hist));
        }
        return;
    }
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The score loads first, bounded by the row length only: the visible
    // count (two dependent scalar loads, which take their own path) arrives
    // meanwhile and masks the keys past it.  Rows are 16-byte aligned: the
    // launcher takes this kernel only for a 16-byte aligned score array whose
    // row length is a multiple of 4.
    const int seq = a.q_seq[t], pos = a.q_pos[t];
    const int max_slots = a.max_slots;
    const float *sc = a.scores + static_cast<int64_t>(t) * max_slots;
    const int wbase = w * 64 * R;
    f32x4 raw[R4];                                // raw[q]: slots wbase + 256q + 4 lane + (0..3)
#pragma unroll
    for (int q = 0; q < R4; q++) {
        // unconditional (a load under a branch costs a branch per load):
        // units past the row re-read its last unit, whose keys lie past the
        // visible count and are masked below
        const int s0 = wbase + 256 * q + 4 * lane;
        raw[q] = *reinterpret_cast<const f32x4 *>(sc + (s0 < max_slots ? s0 : max_slots - 4));
    }
    int n = visible_slots(pos, a.ratio, a.n_slots[seq]);
    n = n < max_slots ? n : max_slots;
    const int k = a.k;
    const int k_eff = n < k ? n : k;
    int32_t *out = a.idx + static_cast<int64_t>(t) * k;
    if (tid == 0) a.len[t] = k_eff;
    if (n <= k) {   // everything visible is selected
        for (int i = tid; i < k; i += THREADS) out[i] = i < n ? i : -1;
        return;
    }

    select_row<THREADS, R, kCandCap>(raw, sc, n, k, [out](int pos, int32_t slot) { out[pos] = slot; },
                                     hist, cand_key, cand_slot, red, sh);
}

// Short lists (up to 2048 visible slots) and rows not 16-byte aligned: the
// exact select over every key, R per thread in the one-key-per-lane layout.
template <int R>
__global__ __launch_bounds__(kTopkThreads) void topk_small_kernel(TopkArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t hist[hist_words<kTopkThreads>()];
    __shared__ int red[2 * kTopkWaves];
    __shared__ int sh[8];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int seq = a.q_seq[t];
    int n = visible_slots(a.q_pos[t], a.ratio, a.n_slots[seq]);
    n = n < a.max_slots ? n : a.max_slots;
    const int k = a.k;
    const int k_eff = n < k ? n : k;
    int32_t *out = a.idx + static_cast<int64_t>(t) * k;
    if (tid == 0) a.len[t] = k_eff;
    if (n <= k) {
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }
    const float *sc = a.scores + static_cast<int64_t>(t) * a.max_slots;
    const int wbase = w * 64 * R;
    uint32_t key[R];
#pragma unroll
    for (int j = 0; j < R; j++) {
        const int s = wbase + 64 * j + lane;
        key[j] = s < n ? order_key(sc[s]) : 0u;
    }
    topk_select_keys<kTopkThreads, R>(key, n, k, [out](int pos, int32_t slot) { out[pos] = slot; },
                                      nullptr, hist, red, sh);
}


// Visible lists longer than the register kernel holds (> 65536 slots, e.g. a
// 1M-token context at ratio 4): the same radix select, re-reading the scores
// from memory each pass, and an ordered write in 1024-slot rounds.
__global__ __launch_bounds__(kTopkThreads) void topk_long_kernel(TopkArgs a) {
    __shared__ uint32_t hist[kTopkWaves][256];
    __shared__ int scan_sh[2 * kTopkWaves];
    __shared__ int sel_sh[2];

    const int t = blockIdx.x;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int seq = a.q_seq[t];
    int n = visible_slots(a.q_pos[t], a.ratio, a.n_slots[seq]);
    n = n < a.max_slots ? n : a.max_slots;
    const int k = a.k;
    const int k_eff = n < k ? n : k;
    int32_t *out = a.idx + static_cast<int64_t>(t) * k;
    const float *sc = a.scores + static_cast<int64_t>(t) * a.max_slots;
    if (tid == 0) a.len[t] = k_eff;
    if (n <= k) {
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }
    uint32_t prefix = 0;
    int remaining = k;
#pragma unroll 1
    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        const uint32_t hi_mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
        for (int i = tid; i < n; i += kTopkThreads) {
            uint32_t kk = order_key(sc[i]);
            if ((kk & hi_mask) == prefix) atomicAdd(&hist[w][(kk >> shift) & 255u], 1u);
        }
        __syncthreads();
        int cnt = 0;
        if (tid < 256)
            for (int ww = 0; ww < kTopkWaves; ww++) cnt += hist[ww][255 - tid];
        const int incl = wave_incl_scan(cnt);
        if (tid < 256 && (tid & 63) == 63) scan_sh[w] = incl;
        __syncthreads();
        if (tid < 256) {
            int before = 0;
#pragma unroll
            for (int ww = 0; ww < 4; ww++) before += ww < w ? scan_sh[ww] : 0;   // tid < 256: w < 4
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
    const uint32_t thr = prefix;
    const int take_eq = remaining;
    int eq_done = 0, sel_done = 0;
    for (int b0 = 0; b0 < n; b0 += kTopkThreads) {
        int i = b0 + tid;
        uint32_t kk = i < n ? order_key(sc[i]) : 0u;
        int gt = (i < n && kk > thr) ? 1 : 0;
        int eq = (i < n && kk == thr) ? 1 : 0;
        int gt_b, eq_b;
        block_scan2(gt, eq, scan_sh, gt_b, eq_b);
        int eq_rank = eq_done + eq_b;
        int before_sel = sel_done + gt_b + (eq_done + eq_b < take_eq ? eq_b : (take_eq > eq_done ? take_eq - eq_done : 0));
        bool sel = gt || (eq && eq_rank < take_eq);
        if (sel) out[before_sel] = i;
        // block totals (scan_sh holds per-wave inclusive totals)
        int tot_gt = 0, tot_eq = 0;
        for (int ww = 0; ww < kTopkWaves; ww++) {
            tot_gt += scan_sh[ww];
            tot_eq += scan_sh[kTopkWaves + ww];
        }
        int eq_taken = eq_done + tot_eq < take_eq ? tot_eq : (take_eq > eq_done ? take_eq - eq_done : 0);
        sel_done += tot_gt + eq_taken;
        eq_done += tot_eq;
        __syncthreads();
    }
    for (int i = k_eff + tid; i < k; i += kTopkThreads) out[i] = -1;
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
    const int per = (a.max_slots + kTopkThreads - 1) / kTopkThreads;
    const bool vec = a.max_slots % 4 == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
    dim3 grid(a.n_q), block(kTopkThreads);
    // the L2 warm-up blocks ride along with the main select kernel only
    const dim3 wgrid(a.warm_q ? static_cast<unsigned>(((a.n_q + 7) & ~7) + a.n_q) : a.n_q);
    if (per <= 1) hipLaunchKernelGGL(topk_small_kernel<1>, grid, block, 0, stream, a);
    else if (per <= 2) hipLaunchKernelGGL(topk_small_kernel<2>, grid, block, 0, stream, a);
    else if (!vec && per <= 16) hipLaunchKernelGGL(topk_small_kernel<16>, grid, block, 0, stream, a);
    else if (!vec && per <= 64) hipLaunchKernelGGL(topk_small_kernel<64>, grid, block, 0, stream, a);
    else if (per <= 4) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 4>), wgrid, block, 0, stream, a);
    else if (per <= 8) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 8>), wgrid, block, 0, stream, a);
    else if (per <= 16) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 16>), wgrid, block, 0, stream, a);
    else if (per <= 32) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 32>), wgrid, block, 0, stream, a);
    else if (per <= 64) hipLaunchKernelGGL((topk_kernel<kTopkThreads, 64>), wgrid, block, 0, stream, a);
    else hipLaunchKernelGGL(topk_long_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace slc
