// topk.hip -- per-query global top-k over the lightning-indexer scores.
//
// Method: "DeepSeek-V4 attention layer types", Indexer / C4A branch: c4a
// computes a global top-k over the indexer scores for every query (the
// IndexCache freq2 page: lists shorter than k are filled with -1).
//
// One workgroup of 1024 threads per query.  The select itself is a radix
// search over order-preserving 32-bit keys: one histogram of 2048 equal bins
// over [min key, max key] finds the bin holding the k-th largest key, its few
// candidates are ranked exactly (key descending, slot ascending), and one
// ordered write places every selected slot in increasing slot order, ties at
// the threshold going to the lower slot.  A prefilter by group maxima first
// cuts the list to a few per cent of it.

#include "slc_internal.hpp"

namespace slc {

// ------------------------------------------------------------------- top-k

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Order-preserving map fp32 -> uint32 (larger score -> larger key); -0 == +0.
// Non-negative floats get the sign bit set, negative ones are inverted
// (the arithmetic shift spreads the sign into the mask): no branch.
__device__ __forceinline__ uint32_t order_key(float s) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

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

// Lanes below this one in the wave whose predicate is set.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
}

constexpr int kHistBits = 11;                 // first histogram: 2048 bins
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistCopies = 1;                // copies of the first histogram (waves w % copies share one)
// words of the shared histogram array: the first histogram, or the crowded
// bin's per-wave 256-bin histograms
constexpr int kHistWords = kHistCopies * kHistBins > kTopkWaves * 256 ? kHistCopies * kHistBins : kTopkWaves * 256;
constexpr int kRankCap = 256;                 // threshold-bin candidates ranked directly

// Top-k of one query's scores by one workgroup of THREADS threads, R keys
// per thread.  Wave w owns slots [64Rw, 64R(w+1)); lane l holds slots
// 64Rw + 64j + l (j < R), so each of its R loads is one coalesced 256-byte
// row of scores and the wave's slots run in (j, lane) order.
//
// Threshold search: one histogram of 2048 equal bins over [kmin, kmax] (bin
// (key - kmin) >> shift) finds the bin holding the k-th largest key.  Its
// candidates (usually a handful) are ranked exactly against each other (key
// descending, slot ascending), which yields the k-th key and how many keys
// equal to it are taken.  A crowded bin falls back to 8-bit radix passes over
// the lower bits of key - kmin.  The ordered write then counts, with wave
// ballots, the selected keys at lower slots.
//
// key: this thread's order keys (entries past n are 0; valid keys never are:
// order_key maps every non-NaN float above 0x007FFFFF); requires n > k.
// Entry i of the list is written out as slot_map[i] (i itself when
// slot_map is null).  Shared memory: hist (kHistWords words,
// 16-byte aligned), red (2 * WAVES ints), sh (8 ints).
//
// range: if non-null, {lo, hi} bound every key from below and above (the
// caller knows them) and the histogram's first kHistCopies * kHistBins words
// are already zero; otherwise the select finds the range and clears them.
template <int THREADS, int R>
__device__ __forceinline__ void topk_select_keys(const uint32_t (&key)[R], int n, int k,
                                                 int32_t *out, const int32_t *slot_map,
                                                 uint32_t *hist, int *red, int *sh,
                                                 const uint32_t *range = nullptr) {
    constexpr int WAVES = THREADS / 64;
    constexpr int BPT = kHistBins / THREADS;
    static_assert(THREADS >= 256 && kHistBins % THREADS == 0, "block size");
    static_assert(WAVES * 256 <= kHistWords && 2 * kRankCap <= kHistWords, "histogram array size");
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wbase = w * 64 * R;

    uint32_t kmin, kmax;
    if (range) {
        kmin = range[0];
        kmax = range[1];
    } else {
#pragma unroll
        for (int i = 0; i < kHistCopies * kHistBins / THREADS; i++) hist[tid + THREADS * i] = 0u;
        kmin = 0xffffffffu;
        kmax = 0u;
#pragma unroll
        for (int j = 0; j < R; j++)
            if (wbase + 64 * j + lane < n) {
                kmin = min(kmin, key[j]);
                kmax = max(kmax, key[j]);
            }
        kmin = wave_umin(kmin);
        kmax = wave_umax(kmax);
        if (lane == 0) {
            red[w] = static_cast<int>(kmin);
            red[WAVES + w] = static_cast<int>(kmax);
        }
        __syncthreads();
        kmin = 0xffffffffu;
        kmax = 0u;
#pragma unroll
        for (int i = 0; i < WAVES; i++) {
            kmin = min(kmin, static_cast<uint32_t>(red[i]));
            kmax = max(kmax, static_cast<uint32_t>(red[WAVES + i]));
        }
    }
    if (kmin == kmax) {   // every entry equal: the lowest ones win
        for (int i = tid; i < k; i += THREADS) out[i] = slot_map ? slot_map[i] : i;
        return;
    }
    // linear bins: key - kmin < 2^hi, bin (key - kmin) >> shift < 2^11
    const int hi = 32 - __clz(kmax - kmin);
    const int shift = hi > kHistBits ? hi - kHistBits : 0;
#pragma unroll
    for (int j = 0; j < R; j++)
        if (wbase + 64 * j + lane < n)
            atomicAdd(&hist[(w % kHistCopies) * kHistBins + ((key[j] - kmin) >> shift)], 1u);
    __syncthreads();

    // thread i owns bins 2047 - BPT*i - b (b < BPT): descending key order
    int cb[BPT], tot = 0;
#pragma unroll
    for (int b = 0; b < BPT; b++) {
        cb[b] = 0;
#pragma unroll
        for (int cp = 0; cp < kHistCopies; cp++) cb[b] += hist[cp * kHistBins + kHistBins - 1 - BPT * tid - b];
        tot += cb[b];
    }
    const int incl = wave_incl_scan(tot);
    if (lane == 63) red[w] = incl;                // red's min/max reads ended before the last barrier
    __syncthreads();
    {
        int before = 0;
#pragma unroll
        for (int i = 0; i < WAVES; i++) before += i < w ? red[i] : 0;
        int run = before + incl - tot;
#pragma unroll
        for (int b = 0; b < BPT; b++) {
            if (run < k && run + cb[b] >= k) {
                sh[0] = kHistBins - 1 - BPT * tid - b;
                sh[1] = run;
                sh[2] = cb[b];
            }
            run += cb[b];
        }
        if (tid == 0) sh[3] = 0;
    }
    __syncthreads();
    const uint32_t bsel = static_cast<uint32_t>(sh[0]);
    const int need = k - sh[1];                   // keys still to take from bin bsel (>= 1)
    const int m = sh[2];                          // keys in bin bsel
    uint32_t prefix = bsel << shift;              // bits [shift, 32) of the bin's keys - kmin
    uint32_t thr;
    int take_eq;
    if (shift == 0) {
        // the bin is one key value
        thr = prefix + kmin;
        take_eq = need;
    } else if (m <= kRankCap) {
        uint32_t *ck = hist;                      // candidates: key, slot
        int *cs = reinterpret_cast<int *>(hist + kRankCap);
#pragma unroll
        for (int j = 0; j < R; j++) {
            const int s = wbase + 64 * j + lane;
            if (s < n && ((key[j] - kmin) >> shift) == bsel) {
                const int pos = atomicAdd(&sh[3], 1);
                ck[pos] = key[j];
                cs[pos] = s;
            }
        }
        __syncthreads();
        if (tid < m) {
            const uint32_t ki = ck[tid];
            const int si = cs[tid];
            int rank = 0, gt = 0;
            // four candidates per (broadcast) LDS read; entries past m are masked
            for (int j0 = 0; j0 < m; j0 += 4) {
                const u32x4 kq = *reinterpret_cast<const u32x4 *>(ck + j0);
                const u32x4 sq = *reinterpret_cast<const u32x4 *>(cs + j0);
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const bool in = j0 + u < m;
                    const uint32_t kj = kq[u];
                    const int sj = static_cast<int>(sq[u]);
                    gt += (in && kj > ki) ? 1 : 0;
                    rank += (in && (kj > ki || (kj == ki && sj < si))) ? 1 : 0;
                }
            }
            if (rank == need - 1) {
                sh[4] = static_cast<int>(ki);
                sh[5] = need - gt;
            }
        }
        __syncthreads();
        thr = static_cast<uint32_t>(sh[4]);
        take_eq = sh[5];
    } else {
        // crowded bin: radix passes over bits [0, shift) of the bin's keys
        uint32_t (*wh)[256] = reinterpret_cast<uint32_t (*)[256]>(hist);   // [WAVES][256]
        int remaining = need;
        int h = shift;
#pragma unroll 1
        while (h > 0) {
            const int width = h < 8 ? h : 8;
            const int sft = h - width;
            for (int i = tid; i < WAVES * 256; i += THREADS) hist[i] = 0u;
            __syncthreads();
            const uint32_t pm = 0xffffffffu << h;
            const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
            for (int j = 0; j < R; j++)
                if (wbase + 64 * j + lane < n && ((key[j] - kmin) & pm) == prefix)
                    atomicAdd(&wh[w][((key[j] - kmin) >> sft) & dmask], 1u);
            __syncthreads();
            int cnt = 0;
            if (tid < 256) {
#pragma unroll
                for (int ww = 0; ww < WAVES; ww++) cnt += wh[ww][255 - tid];
            }
            const int inc = wave_incl_scan(cnt);
            if (tid < 256 && lane == 63) red[w] = inc;
            __syncthreads();
            if (tid < 256) {
                int before = 0;
#pragma unroll
                for (int ww = 0; ww < 4; ww++) before += ww < w ? red[ww] : 0;   // tid < 256: w < 4
                const int excl = before + inc - cnt;
                if (excl < remaining && excl + cnt >= remaining) {
                    sh[6] = 255 - tid;
                    sh[7] = remaining - excl;
                }
            }
            __syncthreads();
            prefix |= static_cast<uint32_t>(sh[6]) << sft;
            remaining = sh[7];
            h = sft;
            __syncthreads();
        }
        thr = prefix + kmin;
        take_eq = remaining;
    }

    // ordered write: a selected slot's place is the number of selected slots
    // below it, i.e. (keys > thr below it) + min(keys == thr below it, take_eq)
    int wg = 0, we = 0;
#pragma unroll
    for (int j = 0; j < R; j++) {
        const bool v = wbase + 64 * j + lane < n;
        wg += __popcll(__ballot(v && key[j] > thr));
        we += __popcll(__ballot(v && key[j] == thr));
    }
    __syncthreads();                              // red / sh reads are done
    if (lane == 0) {
        red[w] = wg;
        red[WAVES + w] = we;
    }
    __syncthreads();
    int g_before = 0, e_before = 0;
#pragma unroll
    for (int i = 0; i < WAVES; i++) {
        g_before += i < w ? red[i] : 0;
        e_before += i < w ? red[WAVES + i] : 0;
    }
#pragma unroll
    for (int j = 0; j < R; j++) {
        const int s = wbase + 64 * j + lane;
        const bool v = s < n;
        const bool gt = v && key[j] > thr, eq = v && key[j] == thr;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        const int gp = g_before + lanes_below(bg);
        const int ep = e_before + lanes_below(be);
        if (gt || (eq && ep < take_eq)) out[gp + (ep < take_eq ? ep : take_eq)] = slot_map ? slot_map[s] : s;
        g_before += __popcll(bg);
        e_before += __popcll(be);
    }
}

// A lower bound of the k-th largest of the values v (G per thread, 0 =
// absent): the floor of the bin, among 2048 equal bins over [min, max], that
// holds the k-th largest; 0 if fewer than k values are present.
// Shared memory as for topk_select_keys, red with 3 * WAVES ints.
template <int THREADS, int G>
__device__ __forceinline__ uint32_t kth_floor(const uint32_t (&v)[G], int k, uint32_t *hist,
                                              int *red, int *sh, uint32_t &largest) {
    constexpr int WAVES = THREADS / 64;
    constexpr int BPT = kHistBins / THREADS;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t vmin = 0xffffffffu, vmax = 0u;
    int cnt = 0;
#pragma unroll
    for (int g = 0; g < G; g++)
        if (v[g]) {
            vmin = min(vmin, v[g]);
            vmax = max(vmax, v[g]);
            cnt++;
        }
    vmin = wave_umin(vmin);
    vmax = wave_umax(vmax);
    cnt = wave_isum(cnt);
#pragma unroll
    for (int i = 0; i < kHistBins / THREADS; i++) hist[tid + THREADS * i] = 0u;
    if (lane == 0) {
        red[w] = static_cast<int>(vmin);
        red[WAVES + w] = static_cast<int>(vmax);
        red[2 * WAVES + w] = cnt;
    }
    __syncthreads();
    vmin = 0xffffffffu;
    vmax = 0u;
    cnt = 0;
#pragma unroll
    for (int i = 0; i < WAVES; i++) {
        vmin = min(vmin, static_cast<uint32_t>(red[i]));
        vmax = max(vmax, static_cast<uint32_t>(red[WAVES + i]));
        cnt += red[2 * WAVES + i];
    }
    largest = vmax;
    // (the early returns are block-uniform; their barrier ends the reads of
    // red above before the caller reuses it)
    if (cnt < k) {
        __syncthreads();
        return 0u;
    }
    if (vmin == vmax) {
        __syncthreads();
        return vmin;
    }
    // linear bins over [vmin, vmax]: (v - vmin) >> shift < 2^11.  (Binning by
    // the top bits below the shared prefix would put a few octaves' worth of
    // values into a few dozen exponent-dominated bins and serialise the
    // atomics on them.)
    const int hi = 32 - __clz(vmax - vmin);
    const int shift = hi > kHistBits ? hi - kHistBits : 0;
#pragma unroll
    for (int g = 0; g < G; g++)
        if (v[g]) atomicAdd(&hist[(v[g] - vmin) >> shift], 1u);
    __syncthreads();
    int cb[BPT], tot = 0;
#pragma unroll
    for (int b = 0; b < BPT; b++) {
        cb[b] = static_cast<int>(hist[kHistBins - 1 - BPT * tid - b]);
        tot += cb[b];
    }
    const int incl = wave_incl_scan(tot);
    if (lane == 63) red[w] = incl;                // red's reads above precede the last barrier
    __syncthreads();
    {
        int run = -tot + incl;
#pragma unroll
        for (int i = 0; i < WAVES; i++) run += i < w ? red[i] : 0;
#pragma unroll
        for (int b = 0; b < BPT; b++) {
            if (run < k && run + cb[b] >= k) sh[0] = kHistBins - 1 - BPT * tid - b;
            run += cb[b];
        }
    }
    __syncthreads();
    return vmin + (static_cast<uint32_t>(sh[0]) << shift);   // the bin's floor
}

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
// (q, lane, e) order.
//
// Prefilter: the four keys of a load are a group; any k group maxima are k
// distinct scores, so the k-th largest maximum (and the floor L of its
// histogram bin) is at most the k-th largest score: no key below L can be
// selected.  The keys >= L (a few per cent of the list) are compacted, in
// slot order, into LDS and the exact select runs on them (kCandCap / THREADS
// per thread).  If more than kCandCap keys pass, the select runs on all keys.
// 1024 threads: with 256 (one wave per SIMD) the phases' latencies were
// exposed (14.4 us on the 64K decode against 10.0), 512 measured no better.
constexpr int kCandCap = 4096;

template <int THREADS, int R>
__global__ __launch_bounds__(THREADS) void topk_kernel(TopkArgs a) {
    static_assert(R >= 4, "16-byte score loads");
    constexpr int R4 = R / 4, WAVES = THREADS / 64;
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistWords];               // 16 KB
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

    uint32_t key[R];                              // key[4q + e]: slot wbase + 256q + 4 lane + e
#pragma unroll
    for (int q = 0; q < R4; q++) {
        const int s0 = wbase + 256 * q + 4 * lane;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t kk = order_key(raw[q][e]);   // computed for every slot, then masked
            key[4 * q + e] = s0 + e < n ? kk : 0u;
        }
    }
    uint32_t gmax[R4];
#pragma unroll
    for (int q = 0; q < R4; q++)
        gmax[q] = max(max(key[4 * q], key[4 * q + 1]), max(key[4 * q + 2], key[4 * q + 3]));
    uint32_t top;                                 // the largest key
    const uint32_t L = kth_floor<THREADS, R4>(gmax, k, hist, red, sh, top);

    // candidates per round and lane: key >= max(L, 1) (valid keys are never
    // 0, so this also excludes the masked slots)
    const uint32_t Lc = L > 1u ? L : 1u;
    int cl[R4], wc = 0;
#pragma unroll
    for (int q = 0; q < R4; q++) {
        cl[q] = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) cl[q] += key[4 * q + e] >= Lc ? 1 : 0;
        wc += cl[q];
    }
    wc = wave_isum(wc);
    if (lane == 0) red[w] = wc;                   // kth_floor's reads of red ended at its last barrier
    __syncthreads();
    int m = 0, run = 0;
#pragma unroll
    for (int i = 0; i < WAVES; i++) {
        m += red[i];
        run += i < w ? red[i] : 0;
    }
    if (m > kCandCap) {
        // crowded: the exact select over every key, in the one-key-per-lane layout
        uint32_t key1[R];
#pragma unroll
        for (int j = 0; j < R; j++) {
            const int s = wbase + 64 * j + lane;
            key1[j] = s < n ? order_key(sc[s]) : 0u;
        }
        __syncthreads();                          // red is reused by the select
        topk_select_keys<THREADS, R>(key1, n, k, out, nullptr, hist, red, sh);
        return;
    }
    // the select's histogram starts cleared (kth_floor is done with it)
#pragma unroll
    for (int i = 0; i < kHistCopies * kHistBins / THREADS; i++) hist[tid + THREADS * i] = 0u;
    // compact the candidates in slot order: round by round, lanes in order,
    // a lane's four slots in order
#pragma unroll
    for (int q = 0; q < R4; q++) {
        const int incl = wave_incl_scan(cl[q]);
        int pos = run + incl - cl[q];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t kk = key[4 * q + e];
            if (kk >= Lc) {
                cand_key[pos] = kk;
                cand_slot[pos] = wbase + 256 * q + 4 * lane + e;
                pos++;
            }
        }
        run += __builtin_amdgcn_readlane(incl, 63);
    }
    __syncthreads();
    if (m == k) {                                 // exactly the candidates
        for (int i = tid; i < k; i += THREADS) out[i] = cand_slot[i];
        return;
    }
    constexpr int Q = kCandCap / THREADS;
    uint32_t ck[Q];
#pragma unroll
    for (int i = 0; i < Q; i++) {
        const int c = w * 64 * Q + 64 * i + lane;
        ck[i] = c < m ? cand_key[c] : 0u;
    }
    // every candidate lies in [L, top]: the select skips its range reduction
    // (L = 0, fewer than k groups: the range is found as usual)
    const uint32_t range[2] = {L, top};
    topk_select_keys<THREADS, Q>(ck, m, k, out, cand_slot, hist, red, sh, L > 0 ? range : nullptr);
}

// Short lists (up to 2048 visible slots) and rows not 16-byte aligned: the
// exact select over every key, R per thread in the one-key-per-lane layout.
template <int R>
__global__ __launch_bounds__(kTopkThreads) void topk_small_kernel(TopkArgs a) {
    __shared__ __attribute__((aligned(16))) uint32_t hist[kHistWords];
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
    topk_select_keys<kTopkThreads, R>(key, n, k, out, nullptr, hist, red, sh);
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
