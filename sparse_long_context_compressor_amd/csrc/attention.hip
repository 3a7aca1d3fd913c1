// attention.hip -- sparse MLA attention in absorbed (MQA) form over the
// sliding window plus the selected compressed slots.
//
// Method: "From MLA to CSA + HCA", Ch.2 (absorbed MLA: every query head
// attends one shared 576-wide latent row per entry, values are the row's
// first 512 dims); "DeepSeek-V4 attention layer types", Indexer / C4A / C128A
// (the kernel takes SWA indices together with compressed top-k indices);
// "DeepseekV4Attention" (devpress), _forward_decode / _forward_prefill.
//
// This file holds the prefill kernel, the merge of decode list splits, the
// decode's split plan and the launchers; the decode kernel itself is in
// decode.hip.
//
// Prefill.  Every attended entry of a query is first resolved through the
// block tables into a physical row (SWA entries e < window are positions
// p-window+1+e, the rest are compressed slot ids).  The rows are then
// gathered chunk by chunk into an LDS tile as bf16 (compressed rows
// dequantised on the way: code * scale; SWA rows too when the SWA pool holds
// fp8 rows, as "From MLA to CSA + HCA" 5.5 describes the V4 SWA cache), with
// later chunks' global loads in flight.  On a tile:
//   S^T = K . Q^T               v_mfma_f32_16x16x32_bf16, one wave per 16
//                               heads, its Q^T in registers
//   online softmax per head     each lane owns one head: no cross-lane rescale
//   O^T += V^T . P^T            the score accumulators' lane layout already is
//                               the P^T operand layout (the MFMA k-order is a
//                               shared permutation of the rows); V^T comes
//                               from the row-major tile via ds_read_tr16_b64,
//                               each wave taking a slice of the output dims
//                               for every head.
// Decode splits.  When a query's list is split across workgroups (decode.hip),
// mla_combine_kernel merges the partial (O, max, sum) states.

#include "slc_internal.hpp"

namespace slc {

namespace {

constexpr int kKPitch = kD + 16;       // bf16 per LDS row: 1184 B (2 mod 4 16-byte units: no bank conflicts for the K and V^T reads)
constexpr int kMaxEntries = SLC_MAX_WINDOW + SLC_MAX_TOPK;
constexpr int kMaxCombineSplits = 8;    // splits the combine kernel merges unrolled

typedef short i16x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) { return f32x2_to_bf16x2(lo, hi); }

// Physical row of attended entry e of query t (-1: skipped).
__device__ __forceinline__ int32_t resolve_entry(const AttnArgs &a, int t, int seq, int p, int ns,
                                                 int e) {
    int64_t r = -1;
    if (e < a.window) {
        int pos = p - a.window + 1 + e;
        if (pos >= 0) r = pool_row(a.swa, seq, pos);
    } else {
        int s = a.cmp_idx[static_cast<int64_t>(t) * a.k + (e - a.window)];
        if (s >= 0 && s < ns) r = pool_row(a.cmp, seq, s);
    }
    return static_cast<int32_t>(r);
}

// Row-wise gather by one producer wave: RPW rows per chunk.  For each row the
// 64 lanes take the 512 nope dims (SWA: 8 bf16 = 16 B per lane; compressed:
// 8 e4m3 codes = 8 B plus that block's scale), then the 64 rope dims of 8 rows
// at a time (lane -> row lane/8, 16-byte unit lane%8).  A row's kind and base
// address are the same for every lane.
// Skipped rows read from this zero page instead of branching around their
// loads: every row issues the same loads, so no load result has to be merged
// at a control-flow join (which would force a wait on each row in turn).
__device__ __attribute__((aligned(256))) uint8_t kZeroPage[2048];   // never written

// F8: the SWA pool holds fp8 rows in the compressed-row layout too.
template <int RPW, bool F8>
struct RowGather {
    u32x4 nope[RPW];        // SWA: 8 bf16; compressed: 8 codes in the low 8 bytes
    float scl[RPW];         // compressed: the lane's 64-dim block scale
    u32x4 rope[RPW / 8];

    // src holds the resolved rows of entries ebase, ebase+1, ...
    __device__ __forceinline__ void load(const AttnArgs &a, const int32_t *src, int ebase, int e0,
                                         int e_end, int pw, int lane) {
        // one LDS read brings this wave's RPW row ids; each is then moved to a
        // scalar register (v_readlane), so row bases are scalar and the loads
        // use a scalar base plus a per-lane offset
        const int eb = __builtin_amdgcn_readfirstlane(e0 + pw * RPW);
        const int my_e = eb + (lane % RPW);
        const int32_t my_row = my_e < e_end ? src[my_e - ebase] : -1;
        const int window = __builtin_amdgcn_readfirstlane(a.window);
#pragma unroll
        for (int j = 0; j < RPW; j++) {
            const int32_t row = __builtin_amdgcn_readlane(my_row, j);
            const bool cmp = eb + j >= window;
            const bool f8 = F8 || cmp;                  // a row in the compressed-row layout
            const int64_t blk = row >> 6, r = row & 63;
            const uint8_t *cbase = reinterpret_cast<const uint8_t *>(cmp ? a.cmp.base : a.swa.base) +
                                   blk * SLC_CMP_BLOCK_BYTES;
            const uint8_t *sbase = reinterpret_cast<const uint8_t *>(a.swa.base) + static_cast<int64_t>(row) * (kD * 2);
            const uint8_t *base = row < 0 ? kZeroPage : (f8 ? cbase : sbase);
            const uint32_t noff = (row >= 0 && f8) ? static_cast<uint32_t>(r * SLC_CMP_ROW_BYTES) + 8u * lane
                                                   : 16u * lane;   // fp8: 16-byte read, low 8 used
            const uint32_t soff = (row >= 0 && f8)
                                      ? static_cast<uint32_t>(SLC_CMP_SCALE_OFFSET + r * 32) + 4u * (lane >> 3)
                                      : 0u;
            nope[j] = *reinterpret_cast<const u32x4 *>(base + noff);
            scl[j] = *reinterpret_cast<const float *>(base + soff);
        }
#pragma unroll
        for (int q = 0; q < RPW / 8; q++) {
            const int jr = 8 * q + (lane >> 3);
            const int e = eb + jr;
            const int part = lane & 7;
            const int32_t row = __shfl(my_row, jr, 64);   // lanes read different rows here
            const uint8_t *pr = kZeroPage + 16 * part;
            if (row >= 0)
                pr = (e >= a.window ? cmp_row_ptr(a.cmp, row) + kDN
                      : F8          ? cmp_row_ptr(a.swa, row) + kDN
                                    : reinterpret_cast<const uint8_t *>(swa_row_ptr(a.swa, row) + kDN)) +
                     16 * part;
            rope[q] = *reinterpret_cast<const u32x4 *>(pr);
        }
    }

    // Dequantise compressed rows (code * scale -> bf16; exact for the
    // power-of-two scales compress writes) and write the rows into the tile.
    // Entries e >= window are compressed rows (skipped ones hold zeros).
    // Half H writes rows [H*RPW/2, (H+1)*RPW/2) and its share of the rope
    // groups, so a chunk can be stored in two steps.
    template <int H>
    __device__ __forceinline__ void store_half(uint16_t *tile, const AttnArgs &a, int e0, int pw,
                                               int lane) const {
        constexpr int J0 = H * RPW / 2, J1 = (H + 1) * RPW / 2;
        constexpr int NQ = RPW / 8, Q0 = H * (NQ / 2), Q1 = H == 0 ? NQ / 2 : NQ;
#pragma unroll
        for (int j = J0; j < J1; j++) {
            u32x4 v = nope[j];
            if (F8 || e0 + pw * RPW + j >= a.window) {
                // e4m3 * scale -> bf16 in one packed conversion per pair; exact for
                // power-of-two scales (the ABI's scale format)
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const float sc = scl[j];
                bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(v[0]), sc, false);
                bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(v[0]), sc, true);
                bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(v[1]), sc, false);
                bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(v[1]), sc, true);
                v = u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                          __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
            }
            *reinterpret_cast<u32x4 *>(tile + (pw * RPW + j) * kKPitch + 8 * lane) = v;
        }
#pragma unroll
        for (int q = Q0; q < Q1; q++)
            *reinterpret_cast<u32x4 *>(tile + (pw * RPW + 8 * q + (lane >> 3)) * kKPitch + kDN +
                                       8 * (lane & 7)) = rope[q];
    }
    __device__ __forceinline__ void store(uint16_t *tile, const AttnArgs &a, int e0, int pw,
                                          int lane) const {
        store_half<0>(tile, a, e0, pw, lane);
        store_half<1>(tile, a, e0, pw, lane);
    }
};

// Q^T as the B operand for 16 heads: lane (g, c) holds head h0 + c, dims 8g + 32s .. +8.
__device__ __forceinline__ void load_q(const AttnArgs &a, int t, int h, int g, bf16x8 (&qb)[kD / 32]) {
    const uint16_t *qp = a.q + (static_cast<int64_t>(t) * a.n_heads + h) * kD + 8 * g;
#pragma unroll
    for (int s = 0; s < kD / 32; s++)
        qb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qp + 32 * s));
}

// Online-softmax update for one head per lane.  x: this lane's logits (log2
// domain, -inf for skipped rows); the row set spans the lane's x and the
// same head's lanes in the other three 16-lane groups.  Writes p = 2^(x-m).
// The reference point m moves only when a logit exceeds it by more than
// kLazyLog2 (p then stays below 2^kLazyLog2, harmless in bf16 / fp32), so
// the O accumulators are rescaled rarely; numerator and denominator share m,
// which keeps the result exact in any case.  Returns the rescale factor.
constexpr float kLazyLog2 = 8.0f;

template <int N>
__device__ __forceinline__ float softmax_update(float (&x)[N], float &m_run, float &l_run,
                                                float (&p)[N]) {
    float cmax = x[0];
#pragma unroll
    for (int i = 1; i < N; i++) cmax = fmaxf(cmax, x[i]);
    cmax = xor32_max(xor16_max(cmax));
    float alpha = 1.f;
    if (cmax > m_run + kLazyLog2) {      // also taken when m_run = -inf and cmax is finite
        alpha = __builtin_amdgcn_exp2f(m_run - cmax);
        m_run = cmax;
    }
    float psum = 0.f;
    if (m_run == -INFINITY) {
#pragma unroll
        for (int i = 0; i < N; i++) p[i] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) {
            p[i] = __builtin_amdgcn_exp2f(x[i] - m_run);
            psum += p[i];
        }
    }
    psum = xor32_sum(xor16_sum(psum));
    l_run = l_run * alpha + psum;
    return alpha;
}

__device__ __forceinline__ void store_out(const AttnArgs &a, int t, int h, int g,
                                          const f32x4 (&o)[kDN / 16], float m_run, float l_run) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t *op = a.out + (static_cast<int64_t>(t) * a.n_heads + h) * kDN + 4 * g;
#pragma unroll
    for (int ct = 0; ct < kDN / 16; ct++)
        *reinterpret_cast<u32x2 *>(op + 16 * ct) =
            u32x2{bf16_pair_rne(o[ct][0] * inv, o[ct][1] * inv),
                  bf16_pair_rne(o[ct][2] * inv, o[ct][3] * inv)};
    if (a.lse && g == 0)
        a.lse[static_cast<int64_t>(t) * a.n_heads + h] =
            l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

constexpr int kPreRows = 32;   // rows per prefill chunk

}  // namespace

// Merge the list splits: with O_s the split's normalised output,
// out = sum_s l_s 2^(m_s - M) O_s / sum_s l_s 2^(m_s - M).
// One thread per (query, head, 8 output columns): one 16-byte load of O and
// one 8-byte load of (m, l) per split.  SN > 0: exactly SN splits, every
// load issued before any is used (no data-dependent branch between them);
// SN = 0: any number, in a loop.
// Grid: ceil(n_q / 8) * 8 * NB blocks of 256 threads, NB = n_heads / 4 per
// query; the blocks of query t share blockIdx % 8 with the decode's
// workgroups of t, so a query's partial states are read on the XCD (and
// through the L2) that wrote them.
constexpr int kCombCols = 8;

template <int SN>
__global__ __launch_bounds__(256) void mla_combine_kernel(AttnArgs a) {
    const int nb = a.n_heads * (kDN / kCombCols) / 256;              // blocks per query
    const int grp = blockIdx.x / (8 * nb), rem = blockIdx.x % (8 * nb);
    const int t = 8 * grp + (rem & 7);
    if (t >= a.n_q) return;                                          // uniform per block
    const int id = (rem >> 3) * 256 + threadIdx.x;                   // within the query
    const int h = id / (kDN / kCombCols);
    const int c8 = id % (kDN / kCombCols);
    const int S = SN > 0 ? SN : a.n_splits;
    auto slot_of = [&](int sp) { return (static_cast<int64_t>(t) * S + sp) * a.n_heads + h; };
    auto ml_of = [&](int64_t slot) { return *reinterpret_cast<const f32x2 *>(a.part_ml + 2 * slot); };
    auto o_of = [&](int64_t slot) {
        return *reinterpret_cast<const u32x4 *>(a.part_o + slot * kDN + kCombCols * c8);
    };
    float M = -INFINITY, L = 0.f;
    float acc[kCombCols] = {};
    auto add = [&](u32x4 v, float wgt) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            acc[2 * j] += __uint_as_float(v[j] << 16) * wgt;
            acc[2 * j + 1] += __uint_as_float(v[j] & 0xffff0000u) * wgt;
        }
    };
    if constexpr (SN > 0) {
        f32x2 ml[SN];
        u32x4 ov[SN];
#pragma unroll
        for (int sp = 0; sp < SN; sp++) {
            ml[sp] = ml_of(slot_of(sp));
            ov[sp] = o_of(slot_of(sp));
        }
#pragma unroll
        for (int sp = 0; sp < SN; sp++) M = ml[sp][1] > 0.f ? fmaxf(M, ml[sp][0]) : M;
#pragma unroll
        for (int sp = 0; sp < SN; sp++) {
            const float wgt = ml[sp][1] > 0.f ? ml[sp][1] * exp2f(ml[sp][0] - M) : 0.f;
            L += wgt;
            add(ov[sp], wgt);
        }
    } else {
        for (int sp = 0; sp < S; sp++) {
            const f32x2 ml = ml_of(slot_of(sp));
            if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
        }
        for (int sp = 0; sp < S; sp++) {
            const f32x2 ml = ml_of(slot_of(sp));
            const float wgt = ml[1] > 0.f ? ml[1] * exp2f(ml[0] - M) : 0.f;
            L += wgt;
            add(o_of(slot_of(sp)), wgt);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *reinterpret_cast<u32x4 *>(a.out + (static_cast<int64_t>(t) * a.n_heads + h) * kDN + kCombCols * c8) =
        u32x4{bf16_pair_rne(acc[0] * inv, acc[1] * inv), bf16_pair_rne(acc[2] * inv, acc[3] * inv),
              bf16_pair_rne(acc[4] * inv, acc[5] * inv), bf16_pair_rne(acc[6] * inv, acc[7] * inv)};
    if (a.lse && c8 == 0)
        a.lse[static_cast<int64_t>(t) * a.n_heads + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// ----------------------------------------------------------------- prefill
// Eight waves: four compute, four gather.  Two LDS tiles alternate: while the
// compute waves work on chunk c (32 rows) in one, the gather waves write
// chunk c + 1 into the other (its loads were issued two chunks ahead).
// Per chunk:
//   scores   compute wave w < NW owns heads 16w..16w+15 of the block: S^T for
//            the chunk's rows, its heads' online softmax, and publishes the
//            P^T operands and rescale factors of its heads in LDS;
//   values   compute wave w owns output dims 128w..128w+127 of every head:
//            each V^T operand, read once with ds_read_tr16_b64, serves the
//            NW head groups' P^T operands (a quarter of the transposing reads
//            that one wave per head group over all 512 dims would need).
// Barriers: one before chunk 0, one between a chunk's scores and its values,
// one between chunks, one before the output (both roles take all of them).
template <int NW, bool F8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_prefill_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ktile[2][kPreRows * kKPitch];
    __shared__ __attribute__((aligned(16))) int32_t src[kMaxEntries + kPreRows];   // -1 past the list
    __shared__ u32x4 pshare[4][64];                 // P^T operands per head group
    __shared__ float ashare[4][16];                 // rescale factor per head
    __shared__ float lshare[4][16];                 // final sum per head

    constexpr int NT = 512;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int t = blockIdx.x;
    const int h0 = 16 * NW * blockIdx.y;            // head block (NW groups of 16)
    const int seq = a.q_seq[t], p = a.q_pos[t];
    const int E = a.window + a.k;
    const int ns = a.k > 0 ? a.n_slots[seq] : 0;

    const int nchunks = (E + kPreRows - 1) / kPreRows;
    for (int e = tid; e < nchunks * kPreRows; e += NT) src[e] = e < E ? resolve_entry(a, t, seq, p, ns, e) : -1;
    __syncthreads();

    if (w >= 4) {
        RowGather<kPreRows / 4, F8> ga, gb;     // chunks 0, 2, 4, ... and 1, 3, 5, ...
        const int pw = __builtin_amdgcn_readfirstlane(w - 4);
        // unconditional loads (past the list: the zero page), so that a
        // buffer's store waits for its own loads only
        ga.load(a, src, 0, 0, E, pw, lane);
        gb.load(a, src, 0, kPreRows, E, pw, lane);
        ga.store(ktile[0], a, 0, pw, lane);
        ga.load(a, src, 0, 2 * kPreRows, E, pw, lane);
        __syncthreads();                                  // chunk 0 in tile 0
        for (int cc = 0; cc < nchunks; cc += 2) {
            // chunk cc + 1 into tile 1 (chunk cc - 1's values are done)
            if (cc + 1 < nchunks) {
                gb.store(ktile[1], a, (cc + 1) * kPreRows, pw, lane);
                gb.load(a, src, 0, (cc + 3) * kPreRows, E, pw, lane);
            }
            __syncthreads();                              // chunk cc: scores -> values
            if (cc + 1 >= nchunks) break;
            __syncthreads();                              // chunk cc done, cc + 1 in tile 1
            if (cc + 2 < nchunks) {
                ga.store(ktile[0], a, (cc + 2) * kPreRows, pw, lane);
                ga.load(a, src, 0, (cc + 4) * kPreRows, E, pw, lane);
            }
            __syncthreads();                              // chunk cc + 1: scores -> values
            if (cc + 2 >= nchunks) break;
            __syncthreads();                              // chunk cc + 1 done, cc + 2 in tile 0
        }
        __syncthreads();                                  // the final sums
        return;
    }

    const bool owner = w < NW;                            // a head group's scores
    bf16x8 qb[kD / 32];
    if (owner) load_q(a, t, h0 + 16 * w + c, g, qb);
    f32x4 o[NW][8];                                       // dims 128w + 16 ct + 4g.., head 16 hg + c
#pragma unroll
    for (int hg = 0; hg < NW; hg++)
#pragma unroll
        for (int ct = 0; ct < 8; ct++) o[hg][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    __syncthreads();                                      // chunk 0 in tile 0
    for (int cc = 0; cc < nchunks; cc++) {
        const int e0 = cc * kPreRows;
        const uint16_t *kt = ktile[cc & 1];
        if (owner) {
            // the rows' ids (-1: skipped or past the list), read ahead of the products
            i32x4 sv[2];
#pragma unroll
            for (int mt = 0; mt < 2; mt++) sv[mt] = *reinterpret_cast<const i32x4 *>(src + e0 + 16 * mt + 4 * g);
            // per row tile, two accumulators (even and odd k-steps), so that
            // consecutive products do not wait for each other
            f32x4 sacc[2];
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
                const uint16_t *kr = kt + (16 * mt + c) * kKPitch + 8 * g;
#pragma unroll
                for (int s = 0; s < kD / 32; s += 2) {
                    bf16x8 k0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kr + 32 * s));
                    bf16x8 k1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kr + 32 * s + 32));
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qb[s], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qb[s + 1], s1, 0, 0, 0);
                }
                sacc[mt] = s0 + s1;
            }
            float x[8], pv[8];
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int i = 0; i < 4; i++) x[4 * mt + i] = sv[mt][i] >= 0 ? sacc[mt][i] * a.sm_scale_log2 : -INFINITY;
            const float alpha = softmax_update<8>(x, m_run, l_run, pv);
            // k = 32 rows: 4g+0..3 then 16+4g+0..3 (same order as the V^T reads)
            pshare[w][lane] = u32x4{bf16_pair_rne(pv[0], pv[1]), bf16_pair_rne(pv[2], pv[3]),
                                    bf16_pair_rne(pv[4], pv[5]), bf16_pair_rne(pv[6], pv[7])};
            if (g == 0) ashare[w][c] = alpha;
        }
        __syncthreads();                                  // the chunk's P^T and factors

        bf16x8 pb[NW];
        float al[NW];
#pragma unroll
        for (int hg = 0; hg < NW; hg++) {
            pb[hg] = __builtin_bit_cast(bf16x8, pshare[hg][lane]);
            al[hg] = ashare[hg][c];
        }
#pragma unroll
        for (int hg = 0; hg < NW; hg++) {
            if (__ballot(al[hg] != 1.f)) {
#pragma unroll
                for (int ct = 0; ct < 8; ct++) o[hg][ct] *= al[hg];
            }
        }
        const uint16_t *v1 = kt + (4 * g + (c >> 2)) * kKPitch + 4 * (c & 3) + 128 * w;
        const uint16_t *v2 = v1 + 16 * kKPitch;
#pragma unroll
        for (int ct = 0; ct < 8; ct++) {
            i16x4 lo = lds_read_tr16(v1 + 16 * ct);
            i16x4 hi = lds_read_tr16(v2 + 16 * ct);
            u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
#pragma unroll
            for (int hg = 0; hg < NW; hg++)
                o[hg][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[hg], o[hg][ct], 0, 0, 0);
        }
        if (cc + 1 < nchunks) __syncthreads();           // chunk cc done, cc + 1 in the other tile
    }

    // the owners' sums (and log-sum-exp) of their heads, then every wave
    // normalises and writes its dims of every head
    if (owner && g == 0) {
        lshare[w][c] = l_run;
        if (a.lse)
            a.lse[static_cast<int64_t>(t) * a.n_heads + h0 + 16 * w + c] =
                l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int hg = 0; hg < NW; hg++) {
        const float l = lshare[hg][c];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t *op = a.out + (static_cast<int64_t>(t) * a.n_heads + h0 + 16 * hg + c) * kDN + 128 * w + 4 * g;
#pragma unroll
        for (int ct = 0; ct < 8; ct++)
            *reinterpret_cast<u32x2 *>(op + 16 * ct) =
                u32x2{bf16_pair_rne(o[hg][ct][0] * inv, o[hg][ct][1] * inv),
                      bf16_pair_rne(o[hg][ct][2] * inv, o[hg][ct][3] * inv)};
    }
}

// Decode split plan (host arithmetic only).  Head groups per workgroup: 2
// (32 heads) when H % 32 == 0, else 1.  The decode moves each split's rows
// into LDS at once and is bound by how fast the compute units pull bytes, so
// the lists are split until about one workgroup runs per CU (256): S =
// ceil(256 / (queries x head blocks)), at most kMaxCombineSplits, and fewer
// while a split would hold under 32 entries.  No split at all when splitting
// would take fewer than kMergeRows entries off each workgroup: the merge (a
// second launch over the partial states) costs more than that saves (the
// 128-row window of 64 queries measured 13.5 us unsplit against 16.5 us in
// two splits plus the merge; one query's 384 entries 16.5 us in 8 splits
// against 18.4 us in 4).  Prefill never splits.
void attention_plan(int n_q, int n_heads, int window, int k, bool decode, int *n_splits,
                    int *rows_per_split, int *head_groups) {
    const int entries = window + k;
    if (!decode) {
        *n_splits = 1;
        *rows_per_split = entries;
        *head_groups = 1;
        return;
    }
    constexpr int kCUs = 256;
    const int ng = n_heads % 32 == 0 ? 2 : 1;
    const int blocks = (n_q > 0 ? n_q : 1) * (n_heads / (16 * ng));
    int sp = (kCUs + blocks - 1) / blocks;
    sp = sp < kMaxCombineSplits ? sp : kMaxCombineSplits;
    while (sp > 1 && entries / sp < 32) sp--;
    constexpr int kMergeRows = 80;
    if (sp > 1 && entries * (sp - 1) < kMergeRows * sp) sp = 1;
    *n_splits = sp;
    *rows_per_split = (entries + sp - 1) / sp;
    *head_groups = ng;
}

hipError_t launch_combine(const AttnArgs &a, hipStream_t stream) {
    // n_heads is a multiple of 16, so a query's threads fill whole blocks
    const unsigned nb = static_cast<unsigned>(a.n_heads * (kDN / kCombCols) / 256);
    const dim3 cgrid(static_cast<unsigned>((a.n_q + 7) / 8) * 8u * nb), cblock(256);
    switch (a.n_splits) {
    case 2: hipLaunchKernelGGL(mla_combine_kernel<2>, cgrid, cblock, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(mla_combine_kernel<3>, cgrid, cblock, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(mla_combine_kernel<4>, cgrid, cblock, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(mla_combine_kernel<5>, cgrid, cblock, 0, stream, a); break;
    case 6: hipLaunchKernelGGL(mla_combine_kernel<6>, cgrid, cblock, 0, stream, a); break;
    case 7: hipLaunchKernelGGL(mla_combine_kernel<7>, cgrid, cblock, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(mla_combine_kernel<8>, cgrid, cblock, 0, stream, a); break;
    default: hipLaunchKernelGGL(mla_combine_kernel<0>, cgrid, cblock, 0, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, bool decode, hipStream_t stream) {
    if (decode) {
        hipError_t e = launch_decode(a, stream);
        if (e != hipSuccess || a.n_splits == 1) return e;
        return launch_combine(a, stream);
    }
    // head blocks of up to four 16-head groups, all blocks alike: the fewest
    // blocks that divide the groups evenly (80 heads: five blocks of 16)
    const int groups = a.n_heads / 16;
    int hb = (groups + 3) / 4;
    while (groups % hb != 0) hb++;
    const int nw = groups / hb;
    dim3 grid(a.n_q, hb);
    if (a.swa_fp8) {
        switch (nw) {
        case 1: hipLaunchKernelGGL((mla_prefill_kernel<1, true>), grid, dim3(512), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((mla_prefill_kernel<2, true>), grid, dim3(512), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((mla_prefill_kernel<3, true>), grid, dim3(512), 0, stream, a); break;
        default: hipLaunchKernelGGL((mla_prefill_kernel<4, true>), grid, dim3(512), 0, stream, a); break;
        }
    } else {
        switch (nw) {
        case 1: hipLaunchKernelGGL((mla_prefill_kernel<1, false>), grid, dim3(512), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((mla_prefill_kernel<2, false>), grid, dim3(512), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((mla_prefill_kernel<3, false>), grid, dim3(512), 0, stream, a); break;
        default: hipLaunchKernelGGL((mla_prefill_kernel<4, false>), grid, dim3(512), 0, stream, a); break;
        }
    }
    return hipGetLastError();
}

}  // namespace slc
