// select.hpp -- the exact per-query top-k select, shared by the top-k
// kernels (topk.hip) and the decode that selects its own list (decode.hip).
//
// Method: "DeepSeek-V4 attention layer types", Indexer / C4A branch: c4a
// computes a global top-k over the indexer scores for every query; lists are
// written in increasing slot order, ties at the threshold going to the lower
// slot, and lists shorter than k are filled with -1 (the IndexCache freq2
// page).
//
// Every function here is called by all THREADS threads of a workgroup
// together (they hold workgroup barriers); their early exits are uniform.
#pragma once

#include "slc_device.hpp"

namespace slc {

// Order-preserving map fp32 -> uint32 (larger score -> larger key); -0 == +0.
// Non-negative floats get the sign bit set, negative ones are inverted
// (the arithmetic shift spreads the sign into the mask): no branch.
__device__ __forceinline__ uint32_t order_key(float s) {
    const uint32_t u = __float_as_uint(s + 0.0f);
    return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

// Lanes below this one in the wave whose predicate is set.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u)));
}

constexpr int kHistBits = 11;                 // first histogram: 2048 bins
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistCopies = 1;                // copies of the first histogram (waves w % copies share one)
// words of the shared histogram array of a THREADS-thread select: the first
// histogram, or the crowded bin's per-wave 256-bin histograms
template <int THREADS>
constexpr int hist_words() {
    return kHistCopies * kHistBins > THREADS / 64 * 256 ? kHistCopies * kHistBins : THREADS / 64 * 256;
}
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
// List entry pos is handed to sink(pos, slot) exactly once for every pos < k,
// slot = slot_map[i] for key i (i itself when slot_map is null).  Shared
// memory: hist (hist_words<THREADS>() words, 16-byte aligned), red (2 * WAVES
// ints), sh (8 ints).
//
// range: if non-null, {lo, hi} bound every key from below and above (the
// caller knows them) and the histogram's first kHistCopies * kHistBins words
// are already zero; otherwise the select finds the range and clears them.
template <int THREADS, int R, class Sink>
__device__ __forceinline__ void topk_select_keys(const uint32_t (&key)[R], int n, int k,
                                                 Sink sink, const int32_t *slot_map,
                                                 uint32_t *hist, int *red, int *sh,
                                                 const uint32_t *range = nullptr) {
    constexpr int WAVES = THREADS / 64;
    constexpr int BPT = kHistBins / THREADS;
    static_assert(THREADS >= 256 && kHistBins % THREADS == 0, "block size");
    static_assert(WAVES * 256 <= hist_words<THREADS>() && 2 * kRankCap <= hist_words<THREADS>(),
                  "histogram array size");
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
        for (int i = tid; i < k; i += THREADS) sink(i, slot_map ? slot_map[i] : i);
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
        if (gt || (eq && ep < take_eq)) sink(gp + (ep < take_eq ? ep : take_eq), slot_map ? slot_map[s] : s);
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

// ------------------------------------------------ selection of a score row
// The whole select on one row of scores held in registers, R per thread in
// the layout of 16-byte loads: raw[q] holds slots wbase + 256 q + 4 lane +
// (0..3), wbase = 64 R w.  n visible slots (n > k), k the list length.
//
// Prefilter: the four keys of a load are a group; any k group maxima are k
// distinct scores, so the k-th largest maximum (and the floor L of its
// histogram bin) is at most the k-th largest score: no key below L can be
// selected.  The keys >= L (a few per cent of the list) are compacted, in
// slot order, into LDS and the exact select runs on them (CAND / THREADS
// per thread).  If more than CAND keys pass, the select runs on all keys,
// re-read from sc in the one-key-per-lane layout.
// Shared memory: hist (hist_words<THREADS>() words), cand_key / cand_slot
// (CAND each), red (3 * WAVES ints), sh (8 ints).
template <int THREADS, int R, int CAND, class Sink>
__device__ __forceinline__ void select_row(const f32x4 (&raw)[R / 4], const float *sc, int n, int k,
                                           Sink sink, uint32_t *hist, uint32_t *cand_key,
                                           int32_t *cand_slot, int *red, int *sh) {
    static_assert(R >= 4 && R % 4 == 0, "16-byte score loads");
    static_assert(CAND % THREADS == 0, "candidates per thread");
    constexpr int R4 = R / 4, WAVES = THREADS / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wbase = w * 64 * R;
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
    if (m > CAND) {
        // crowded: the exact select over every key, in the one-key-per-lane layout
        uint32_t key1[R];
#pragma unroll
        for (int j = 0; j < R; j++) {
            const int s = wbase + 64 * j + lane;
            key1[j] = s < n ? order_key(sc[s]) : 0u;
        }
        __syncthreads();                          // red is reused by the select
        topk_select_keys<THREADS, R>(key1, n, k, sink, nullptr, hist, red, sh);
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
        for (int i = tid; i < k; i += THREADS) sink(i, cand_slot[i]);
        return;
    }
    constexpr int Q = CAND / THREADS;
    uint32_t ck[Q];
#pragma unroll
    for (int i = 0; i < Q; i++) {
        const int c = w * 64 * Q + 64 * i + lane;
        ck[i] = c < m ? cand_key[c] : 0u;
    }
    // every candidate lies in [L, top]: the select skips its range reduction
    // (L = 0, fewer than k groups: the range is found as usual)
    const uint32_t range[2] = {L, top};
    topk_select_keys<THREADS, Q>(ck, m, k, sink, cand_slot, hist, red, sh, L > 0 ? range : nullptr);
}

}  // namespace slc
