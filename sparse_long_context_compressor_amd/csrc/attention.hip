// attention.hip -- sparse MLA attention in absorbed (MQA) form over the
// sliding window plus the selected compressed slots.
//
// Method: "From MLA to CSA + HCA", Ch.2 (absorbed MLA: every query head
// attends one shared 576-wide latent row per entry, values are the row's
// first 512 dims); "DeepSeek-V4 attention layer types", Indexer / C4A / C128A
// (the kernel takes SWA indices together with compressed top-k indices);
// "DeepseekV4Attention" (devpress), _forward_decode / _forward_prefill.
//
// Common pieces.  Every attended entry of a query is first resolved through
// the block tables into a physical row (SWA entries e < window are positions
// p-window+1+e, the rest are compressed slot ids); the rows are then gathered
// chunk by chunk into an LDS tile as bf16 (compressed rows dequantised on the
// way: code * scale; SWA rows too when the SWA pool holds fp8 rows, as "From
// MLA to CSA + HCA" 5.5 describes the V4 SWA cache), with the next chunk's
// global loads in flight while the
// current chunk is computed.  On the tile, per wave and 16 heads:
//   S^T = K . Q^T               v_mfma_f32_16x16x32_bf16, Q^T held in registers
//   online softmax per head     each lane owns one head: no cross-lane rescale
//   O^T += V^T . P^T            the score accumulators' lane layout already is
//                               the P^T operand layout (the MFMA k-order is a
//                               shared permutation of the rows), and V^T comes
//                               from the row-major tile via ds_read_tr16_b64.
//
// Decode (few queries, long lists): one workgroup per (query, 16-head group,
// list split); its four waves take 16 rows each of every 64-row chunk and
// merge their softmax states through LDS.  Head groups of one query are
// numbered so that they land on the same XCD and share its L2 for the rows.
// When a query's list is split across workgroups, a combine kernel merges
// the partial (O, max, sum) states.  Prefill (many queries): one workgroup per
// query token; its waves are the head groups and share each 32-row tile.

#include "slc_internal.hpp"

namespace slc {

namespace {

constexpr int kKPitch = kD + 8;        // bf16 per LDS row: 1168 B, spreads banks
constexpr int kMaxEntries = SLC_MAX_WINDOW + SLC_MAX_TOPK;
constexpr int kDecMaxEntries = 1024;   // list entries one decode workgroup resolves
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
        alpha = exp2f(m_run - cmax);
        m_run = cmax;
    }
    float psum = 0.f;
    if (m_run == -INFINITY) {
#pragma unroll
        for (int i = 0; i < N; i++) p[i] = 0.f;
    } else {
#pragma unroll
        for (int i = 0; i < N; i++) {
            p[i] = exp2f(x[i] - m_run);
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

constexpr int kDecRows = 64;   // rows per decode chunk (16 per consumer wave)
static_assert(kDecMaxEntries % kDecRows == 0, "a chunk's list entries lie within the resolved list");
// LDS pitch (bf16) of the decode's output staging rows (128 dims of one
// head): 68 words, so the 8-byte writes of 32 lanes (16 heads x 2 dim
// quads) fall on distinct banks
constexpr int kOutPitch = 128 + 8;
constexpr int kPreRows = 32;   // rows per prefill chunk

// Scores of one wave's score block: 16*NR rows of a chunk (tile row row0 =
// list entry e0) for the wave's 16 heads, S^T = K . Q^T, scaled to the log2
// domain; entries at or past e_end and skipped rows (src: entries counted
// from e_begin -> physical rows, -1 = skipped) give -inf.  x[4rt + i] is
// row 16rt + 4g + i for head c.
template <int NR>
__device__ __forceinline__ void score_rows(const uint16_t *tile, int row0, int e0, int e_begin,
                                           int e_end, const int32_t *src,
                                           const bf16x8 (&qb)[kD / 32], float sm_scale_log2,
                                           float (&x)[4 * NR], int g, int c) {
    // a scheduling region of its own: the LDS-read and MFMA groups pinned
    // below must not interleave with neighbouring work
    __builtin_amdgcn_sched_barrier(0);
    // validity of the lane's rows 16rt + 4g + i (issued before the MFMAs need
    // them): four consecutive, 16-byte aligned entries per row tile, read
    // unconditionally (a chunk's entries lie within src even past e_end) and
    // masked after
    int32_t rv[4 * NR];
#pragma unroll
    for (int rt = 0; rt < NR; rt++) {
        const int e = e0 + 16 * rt + 4 * g;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(src + (e - e_begin));
#pragma unroll
        for (int i = 0; i < 4; i++) rv[4 * rt + i] = e + i < e_end ? static_cast<int32_t>(v[i]) : -1;
    }
    // S^T per 16-row tile: software-pipelined LDS reads (group i+1 in
    // flight while group i feeds the MFMAs), two accumulator chains; the
    // order is pinned with scheduling group barriers
    f32x4 sacc[NR];
#pragma unroll
    for (int rt = 0; rt < NR; rt++) {
        const uint16_t *kr = tile + (row0 + 16 * rt + c) * kKPitch + 8 * g;
        f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
        constexpr int G = 3, NRR = kD / 32 / G;   // 6 groups of 3 k-steps
        bf16x8 ka[2][G];
        auto rd = [&](int gi, int b) {
#pragma unroll
            for (int u = 0; u < G; u++)
                ka[b][u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kr + 32 * (gi * G + u)));
            __builtin_amdgcn_sched_group_barrier(0x100, G, 0);
        };
        auto mm = [&](int gi, int b) {
#pragma unroll
            for (int u = 0; u < G; u++) {
                if (u & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[b][u], qb[gi * G + u], s1, 0, 0, 0);
                else s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[b][u], qb[gi * G + u], s0, 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, G, 0);
        };
        rd(0, 0);
#pragma unroll
        for (int gi = 0; gi < NRR; gi++) {
            if (gi + 1 < NRR) rd(gi + 1, (gi + 1) & 1);
            mm(gi, gi & 1);
        }
        sacc[rt] = s0 + s1;
    }
#pragma unroll
    for (int rt = 0; rt < NR; rt++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            x[4 * rt + i] = rv[4 * rt + i] >= 0 ? sacc[rt][i] * sm_scale_log2 : -INFINITY;
    __builtin_amdgcn_sched_barrier(0);
}

// O^T += V^T . P^T for one wave's 128 output dims (dims 128w + 16d + 4g + i
// in o[d][hg], lane (g, c): head 16hg + c) over all 64 rows of a chunk, for
// every head group.  pl[hg][j][lane] holds the P^T operand of the chunk's
// k-step j (rows 32j .. 32j+31, in the order rows 4g+i, then 16+4g+i), which
// the score waves wrote; the V^T operand is read transposed from the tile in
// the same row order, once per workgroup.
template <int NG>
__device__ __forceinline__ void pv_rows(const uint16_t *tile, const u32x4 (*pl)[2][64],
                                        f32x4 (&o)[8][NG], int w, int g, int c, int lane) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pb[2][NG];
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int hg = 0; hg < NG; hg++) pb[j][hg] = __builtin_bit_cast(bf16x8, pl[hg][j][lane]);
    const uint16_t *vr = tile + (4 * g + (c >> 2)) * kKPitch + 4 * (c & 3) + 128 * w;
    // four groups (k-step j, dims half dh) of four 16-dim tiles; group i+1's
    // reads are in flight while group i feeds the MFMAs
    constexpr int G = 4;
    i16x4 va[2][G], vb[2][G];
    auto rd = [&](int gi, int b) {
        const int j = gi >> 1, dh = gi & 1;
#pragma unroll
        for (int u = 0; u < G; u++) {
            va[b][u] = lds_read_tr16(vr + 32 * j * kKPitch + 16 * (G * dh + u));
            vb[b][u] = lds_read_tr16(vr + (32 * j + 16) * kKPitch + 16 * (G * dh + u));
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * G, 0);
    };
    auto mm = [&](int gi, int b) {
        const int j = gi >> 1, dh = gi & 1;
#pragma unroll
        for (int u = 0; u < G; u++) {
            const u32x2 l2 = __builtin_bit_cast(u32x2, va[b][u]), h2 = __builtin_bit_cast(u32x2, vb[b][u]);
            const bf16x8 vv = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
#pragma unroll
            for (int hg = 0; hg < NG; hg++)
                o[G * dh + u][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[j][hg], o[G * dh + u][hg], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, G * NG, 0);
    };
    rd(0, 0);
#pragma unroll
    for (int gi = 0; gi < 4; gi++) {
        if (gi + 1 < 4) rd(gi + 1, (gi + 1) & 1);
        mm(gi, gi & 1);
    }
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

// ------------------------------------------------------------------ decode
// One workgroup per (query, block of 16*NG heads, list split); 512 threads.
// Waves 4..7 gather 64-row chunks into two LDS tiles (chunk c+1 is stored
// and chunk c+2 is in flight while the consumers compute chunk c; one barrier
// per chunk).  Waves 0..3 compute: with NG = 1 each takes 16 rows of every
// chunk for the block's 16 heads; with NG = 2 wave w takes head group w & 1
// and rows 32*(w >> 1) .. +31, so every gathered row serves 32 heads (half
// the row traffic of 16-head blocks).  The consumers then merge their
// softmax states through LDS.  (A 64-head variant, each wave on every row of
// its own head group with no merge, measured about 1 us slower on the 64K
// decode: its workgroups load twice the Q and its 8-way combine reads twice
// the partials.)
template <int NG, bool F8>
__global__ __launch_bounds__(512) void mla_decode_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ktile[2][kDecRows * kKPitch];
    static_assert(4 * 16 * NG * kOutPitch <= kDecRows * kKPitch, "tile 0 stages the output rows");
    __shared__ __attribute__((aligned(16))) int32_t src[kDecMaxEntries];
    __shared__ __attribute__((aligned(16))) u32x4 pl[NG][2][64];   // P^T operands [head group][k-step][lane]
    __shared__ float cm[4][16], lp[4][16];              // score waves' chunk maxima, row sums

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const bool producer = w >= 4;

    // The prologue's kernel arguments in one round of loads, before anything
    // branches on them (left alone, the compiler spreads them over several
    // dependent rounds at the start, where each costs a full load latency).
    const int32_t *q_seq_p = a.q_seq, *q_pos_p = a.q_pos, *n_slots_p = a.n_slots;
    const int32_t *cmp_idx_p = a.cmp_idx, *swa_tab = a.swa.block_table, *cmp_tab = a.cmp.block_table;
    const int swa_stride = a.swa.table_stride, cmp_stride = a.cmp.table_stride;
    const int64_t swa_nb = a.swa.n_blocks, cmp_nb = a.cmp.n_blocks;
    const int window = a.window, kk = a.k, n_q = a.n_q, rps = a.rows_per_split;
    const int HB = a.n_heads / (16 * NG), S = a.n_splits;
    __asm__ volatile("" ::"s"(q_seq_p), "s"(q_pos_p), "s"(n_slots_p), "s"(cmp_idx_p), "s"(swa_tab),
                     "s"(cmp_tab), "s"(swa_stride), "s"(cmp_stride), "s"(swa_nb), "s"(cmp_nb),
                     "s"(window), "s"(kk), "s"(n_q), "s"(rps), "s"(HB), "s"(S));

    // blocks with equal blockIdx % 8 run on one XCD: give all (head block,
    // split) blocks of a query the same residue, so they share its L2
    const int per_group = 8 * HB * S;
    const int grp = blockIdx.x / per_group, rem = blockIdx.x % per_group;
    const int t = 8 * grp + (rem & 7);
    const int hb = (rem >> 3) % HB, split = (rem >> 3) / HB;
    const int tc = t < n_q ? t : 0;                     // for the prologue's loads (n_q >= 1)

    const int hgw = NG == 2 ? (w & 1) : 0;
    const int row0 = NG == 2 ? 32 * ((w >> 1) & 1) : 16 * (w & 3);   // first chunk row of this wave
    const int E = window + kk;
    const int e_begin = split * rps;
    int e_end = e_begin + rps;
    e_end = e_end < E ? e_end : E;
    const int nchunks = e_end > e_begin ? (e_end - e_begin + kDecRows - 1) / kDecRows : 0;

    // The row list first, in two rounds of loads with no branch between them:
    // the compressed entries' slot ids need only t and are loaded with the
    // query's sequence and position; then every entry's block-table entry
    // (one load each, from the SWA or the compressed table) and the
    // sequence's slot count.  An entry with nothing to look up loads a valid
    // dummy address instead.  The split plan keeps e_end - e_begin within
    // kDecMaxEntries.
    constexpr int kResIt = kDecMaxEntries / 512;
    int32_t slot_id[kResIt];
#pragma unroll
    for (int i = 0; i < kResIt; i++) {
        const int e = e_begin + tid + 512 * i;
        const bool cmpe = e < e_end && e >= window;
        slot_id[i] = *(cmpe ? cmp_idx_p + static_cast<int64_t>(tc) * kk + (e - window) : q_seq_p);
    }
    const int seq = q_seq_p[tc], p = q_pos_p[tc];
    if (t >= n_q) return;
    int32_t pb[kResIt];
    int64_t lrow[kResIt];
    bool look[kResIt];
#pragma unroll
    for (int i = 0; i < kResIt; i++) {
        const int e = e_begin + tid + 512 * i;
        const bool swa = e < window;
        lrow[i] = swa ? static_cast<int64_t>(p - window + 1 + e) : static_cast<int64_t>(slot_id[i]);
        const int64_t lb = lrow[i] >> 6;
        look[i] = e < e_end && lrow[i] >= 0 && lb < (swa ? swa_stride : cmp_stride);
        const int32_t *tab = swa ? swa_tab + static_cast<int64_t>(seq) * swa_stride
                                 : cmp_tab + static_cast<int64_t>(seq) * cmp_stride;
        pb[i] = *(look[i] ? tab + lb : q_seq_p);
    }
    const int ns = *(kk > 0 ? n_slots_p + seq : q_seq_p);   // read only where kk > 0
#pragma unroll
    for (int i = 0; i < kResIt; i++) {
        const bool swa = e_begin + tid + 512 * i < window;
        pb[i] = look[i] && pb[i] >= 0 && pb[i] < (swa ? swa_nb : cmp_nb) && (swa || lrow[i] < ns)
                    ? pb[i] * kBR + static_cast<int32_t>(lrow[i] & (kBR - 1)) : -1;
    }
#pragma unroll
    for (int i = 0; i < kResIt; i++) {
        const int e = e_begin + tid + 512 * i;
        if (e < e_end) src[e - e_begin] = pb[i];
    }
    __syncthreads();

    // The block's 16*NG query heads are one contiguous run of q.  The
    // consumers load it once, coalesced (every 128-byte line by one request;
    // per-head operand loads would request each line four times), into tile 1,
    // which is free until chunk 1 is stored; after one barrier (the producers
    // take it before their first store) each wave reads its head group's
    // operands from there, rows at the K tile's pitch.
    constexpr int kQUnits = 16 * NG * kD / 8;            // 16-byte units
    constexpr int kQIt = (kQUnits + 255) / 256;
    if (!producer) {
        const uint16_t *qsrc = a.q + (static_cast<int64_t>(t) * a.n_heads + 16 * NG * hb) * kD;
        u32x4 qv[kQIt];
#pragma unroll
        for (int i = 0; i < kQIt; i++) {
            const int u = tid + 256 * i;
            if (u < kQUnits) qv[i] = *reinterpret_cast<const u32x4 *>(qsrc + 8 * u);
        }
#pragma unroll
        for (int i = 0; i < kQIt; i++) {
            const int u = tid + 256 * i;
            if (u < kQUnits)
                *reinterpret_cast<u32x4 *>(&ktile[1][(u / (kD / 8)) * kKPitch + 8 * (u % (kD / 8))]) = qv[i];
        }
    }

    if (producer) {
        // Chunk c goes to tile c & 1.  Chunk c+1 is stored in two halves
        // while the consumers work on chunk c (one beside its scores, one
        // beside its value products) and chunk c+2 is in flight.  The loads
        // are issued unconditionally (chunks past the list read the zero
        // page): with the same number of loads in flight on every path,
        // storing one buffer waits for that buffer's loads only.  The
        // producers take every barrier the consumers take.
        RowGather<kDecRows / 4, F8> ga, gb;
        const int pw = __builtin_amdgcn_readfirstlane(w - 4);
        ga.load(a, src, e_begin, e_begin, e_end, pw, lane);
        __syncthreads();                                // the consumers' Q is in tile 1
        // chunk 1 only now: issued with chunk 0 and Q, its loads delayed both
        // in the CU's in-order memory pipeline
        gb.load(a, src, e_begin, e_begin + kDecRows, e_end, pw, lane);
        if (nchunks > 0) ga.store(ktile[0], a, e_begin, pw, lane);
        for (int ci = 0; ci < nchunks; ci += 2) {
            const int e0 = e_begin + ci * kDecRows;
            const bool more1 = ci + 1 < nchunks, more2 = ci + 2 < nchunks;
            __syncthreads();                            // chunk ci ready in tile 0
            ga.load(a, src, e_begin, e0 + 2 * kDecRows, e_end, pw, lane);
            // tile 1 last held chunk ci-1 (or Q), whose readers passed the barrier above
            __syncthreads();                            // the chunk maxima
            if (more1) gb.template store_half<0>(ktile[1], a, e0 + kDecRows, pw, lane);
            __syncthreads();                            // the chunk's probabilities
            if (more1) gb.template store_half<1>(ktile[1], a, e0 + kDecRows, pw, lane);
            if (!more1) break;
            __syncthreads();                            // chunk ci+1 ready in tile 1
            gb.load(a, src, e_begin, e0 + 3 * kDecRows, e_end, pw, lane);
            __syncthreads();                            // the chunk maxima
            if (more2) ga.template store_half<0>(ktile[0], a, e0 + 2 * kDecRows, pw, lane);
            __syncthreads();                            // the chunk's probabilities
            if (more2) ga.template store_half<1>(ktile[0], a, e0 + 2 * kDecRows, pw, lane);
        }
        __syncthreads();                                // the consumers' row sums
        return;
    }

    __syncthreads();                                    // Q staged in tile 1
    bf16x8 qb[kD / 32];                                 // Q^T operands: head 16*hgw + c, dims 8g + 32s
    {
        const uint16_t *qs = &ktile[1][(16 * hgw + c) * kKPitch + 8 * g];
#pragma unroll
        for (int s = 0; s < kD / 32; s++) qb[s] = *reinterpret_cast<const bf16x8 *>(qs + 32 * s);
    }
    // Score wave w covers head group hgw and chunk rows row0 .. row0+16NG-1;
    // for the value products wave w takes output dims 128w .. 128w+127 of
    // every head of the block.  All waves keep the same softmax reference
    // per head (m_run), moved lazily by the largest score of a chunk, so the
    // probabilities of different score waves add up in one accumulator.
    constexpr int NB = 4 / NG;                          // score waves per head group
    f32x4 o[8][NG];
#pragma unroll
    for (int d = 0; d < 8; d++)
#pragma unroll
        for (int hg = 0; hg < NG; hg++) o[d][hg] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[NG];
#pragma unroll
    for (int hg = 0; hg < NG; hg++) m_run[hg] = -INFINITY;
    float l_part = 0.f;                                 // this wave's rows' share of its head's sum

    for (int ci = 0; ci < nchunks; ci++) {
        __syncthreads();                                // chunk ci is in tile ci & 1
        const uint16_t *tile = ktile[ci & 1];
        float x[4 * NG];
        score_rows<NG>(tile, row0, e_begin + ci * kDecRows + row0, e_begin, e_end, src, qb,
                       a.sm_scale_log2, x, g, c);
        float cmax = x[0];
#pragma unroll
        for (int i = 1; i < 4 * NG; i++) cmax = fmaxf(cmax, x[i]);
        cmax = xor32_max(xor16_max(cmax));
        if (g == 0) cm[w][c] = cmax;
        __syncthreads();                                // every score wave's chunk maximum
        float alpha[NG];
        bool rescale[NG];
#pragma unroll
        for (int hg = 0; hg < NG; hg++) {
            float cx = -INFINITY;
#pragma unroll
            for (int r = 0; r < NB; r++) cx = fmaxf(cx, cm[hg + NG * r][c]);
            alpha[hg] = 1.f;
            rescale[hg] = false;
            if (cx > m_run[hg] + kLazyLog2) {           // also taken when m_run = -inf and cx is finite
                rescale[hg] = m_run[hg] != -INFINITY;   // O holds something to rescale
                alpha[hg] = exp2f(m_run[hg] - cx);
                m_run[hg] = cx;
            }
        }
        const float mr = (NG == 2 && hgw == 1) ? m_run[NG - 1] : m_run[0];
        const float am = (NG == 2 && hgw == 1) ? alpha[NG - 1] : alpha[0];
        float pv[4 * NG], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4 * NG; i++) {
            pv[i] = mr == -INFINITY ? 0.f : exp2f(x[i] - mr);
            psum += pv[i];
        }
        psum = xor32_sum(xor16_sum(psum));
        l_part = l_part * am + psum;
        // the P^T operand of k-step w >> 1 (rows 4g+i, then 16+4g+i)
        if constexpr (NG == 2) {
            pl[hgw][w >> 1][lane] = u32x4{bf16_pair_rne(pv[0], pv[1]), bf16_pair_rne(pv[2], pv[3]),
                                          bf16_pair_rne(pv[4], pv[5]), bf16_pair_rne(pv[6], pv[7])};
        } else {
            // score wave w holds rows 16w .. 16w+15: one half of k-step w >> 1
            *reinterpret_cast<u32x2 *>(reinterpret_cast<uint32_t *>(&pl[0][w >> 1][lane]) + 2 * (w & 1)) =
                u32x2{bf16_pair_rne(pv[0], pv[1]), bf16_pair_rne(pv[2], pv[3])};
        }
#pragma unroll
        for (int hg = 0; hg < NG; hg++)
            if (__ballot(rescale[hg] && alpha[hg] != 1.f)) {
#pragma unroll
                for (int d = 0; d < 8; d++) o[d][hg] *= alpha[hg];
            }
        __syncthreads();                                // the chunk's probabilities
        pv_rows<NG>(tile, pl, o, w, g, c, lane);
    }

    // ---- the heads' sums, then this wave's 128 output dims ----
    if (g == 0) lp[w][c] = l_part;
    __syncthreads();                                    // every wave is past its last chunk
    float L[NG], inv[NG];
#pragma unroll
    for (int hg = 0; hg < NG; hg++) {
        L[hg] = 0.f;
#pragma unroll
        for (int r = 0; r < NB; r++) L[hg] += lp[hg + NG * r][c];
        inv[hg] = L[hg] > 0.f ? 1.f / L[hg] : 0.f;
    }
    // O / L as bf16: the output, or with list splits the partial state
    // [t][split][h] (each value at most the largest |V| of the split's rows)
    // plus M and L in fp32.  The rows go through LDS (tile 0 is free now,
    // each wave in its own region; a wave's LDS operations complete in
    // order) so that each store writes 256 contiguous bytes of one head.
    uint16_t *stg = &ktile[0][0] + w * (16 * NG) * kOutPitch;
#pragma unroll
    for (int hg = 0; hg < NG; hg++)
#pragma unroll
        for (int d = 0; d < 8; d++)
            *reinterpret_cast<u32x2 *>(stg + (16 * hg + c) * kOutPitch + 16 * d + 4 * g) =
                u32x2{bf16_pair_rne(o[d][hg][0] * inv[hg], o[d][hg][1] * inv[hg]),
                      bf16_pair_rne(o[d][hg][2] * inv[hg], o[d][hg][3] * inv[hg])};
    __asm__ volatile("" ::: "memory");
    const int h0 = 16 * NG * hb;                        // the block's first head
    const int64_t row0_out = S == 1 ? static_cast<int64_t>(t) * a.n_heads + h0
                                    : (static_cast<int64_t>(t) * S + split) * a.n_heads + h0;
    uint16_t *dst = (S == 1 ? a.out : a.part_o) + row0_out * kDN + 128 * w;
#pragma unroll
    for (int it = 0; it < 4 * NG; it++) {
        const int hh = 4 * it + (lane >> 4), col = 8 * (lane & 15);
        *reinterpret_cast<u32x4 *>(dst + static_cast<int64_t>(hh) * kDN + col) =
            *reinterpret_cast<const u32x4 *>(stg + hh * kOutPitch + col);
    }
    if (w == 0 && g == 0) {
#pragma unroll
        for (int hg = 0; hg < NG; hg++) {
            const int64_t hrow = row0_out + 16 * hg + c;
            if (S == 1) {
                if (a.lse)
                    a.lse[hrow] = L[hg] > 0.f ? (m_run[hg] + log2f(L[hg])) * kLn2 : -INFINITY;
            } else {
                a.part_ml[2 * hrow] = m_run[hg];
                a.part_ml[2 * hrow + 1] = L[hg];
            }
        }
    }
}

// Merge the list splits: with O_s the split's normalised output,
// out = sum_s l_s 2^(m_s - M) O_s / sum_s l_s 2^(m_s - M).
// One thread per (query, head, 8 output columns): one 16-byte load of O and
// one 8-byte load of (m, l) per split.  SN > 0: exactly SN splits, every
// load issued before any is used (no data-dependent branch between them);
// SN = 0: any number, in a loop.
constexpr int kCombCols = 8;

template <int SN>
__global__ __launch_bounds__(256) void mla_combine_kernel(AttnArgs a) {
    const int64_t id = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t per_q = static_cast<int64_t>(a.n_heads) * (kDN / kCombCols);
    if (id >= per_q * a.n_q) return;
    const int t = static_cast<int>(id / per_q);
    const int h = static_cast<int>((id % per_q) / (kDN / kCombCols));
    const int c8 = static_cast<int>(id % (kDN / kCombCols));
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
// NW + 4 waves: waves 0..NW-1 compute (wave w: heads 16w..16w+15 of the block,
// all rows of each 32-row chunk), four more waves gather the next chunk.
template <int NW, bool F8>
__global__ __launch_bounds__((NW + 4) * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_prefill_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ktile[kPreRows * kKPitch];
    __shared__ int32_t src[kMaxEntries];

    constexpr int NT = (NW + 4) * 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int t = blockIdx.x;
    const int h0 = 64 * blockIdx.y;                 // head block (up to 64 heads)
    const int seq = a.q_seq[t], p = a.q_pos[t];
    const int E = a.window + a.k;
    const int ns = a.k > 0 ? a.n_slots[seq] : 0;

    for (int e = tid; e < E; e += NT) src[e] = resolve_entry(a, t, seq, p, ns, e);
    __syncthreads();

    if (w >= NW) {
        RowGather<kPreRows / 4, F8> ga, gb;
        const int pw = __builtin_amdgcn_readfirstlane(w - NW);
        // unconditional loads (past the list: the zero page), so that a
        // buffer's store waits for its own loads only
        ga.load(a, src, 0, 0, E, pw, lane);
        gb.load(a, src, 0, kPreRows, E, pw, lane);
        for (int e0 = 0; e0 < E; e0 += 2 * kPreRows) {
            if (e0 != 0) __syncthreads();
            ga.store(ktile, a, e0, pw, lane);
            __syncthreads();
            ga.load(a, src, 0, e0 + 2 * kPreRows, E, pw, lane);
            if (e0 + kPreRows < E) {
                __syncthreads();
                gb.store(ktile, a, e0 + kPreRows, pw, lane);
                __syncthreads();
            }
            gb.load(a, src, 0, e0 + 3 * kPreRows, E, pw, lane);
        }
        return;
    }

    const int h = h0 + 16 * w + c;
    bf16x8 qb[kD / 32];
    load_q(a, t, h, g, qb);
    f32x4 o[kDN / 16];
#pragma unroll
    for (int ct = 0; ct < kDN / 16; ct++) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int e0 = 0; e0 < E; e0 += kPreRows) {
        if (e0 != 0) __syncthreads();
        __syncthreads();

        f32x4 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint16_t *kr = ktile + (16 * mt + c) * kKPitch + 8 * g;
#pragma unroll
            for (int s = 0; s < kD / 32; s++) {
                bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(kr + 32 * s));
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[s], sacc[mt], 0, 0, 0);
            }
        }
        float x[8], pv[8];
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                int e = e0 + 16 * mt + 4 * g + i;
                x[4 * mt + i] = (e < E && src[e] >= 0) ? sacc[mt][i] * a.sm_scale_log2 : -INFINITY;
            }
        const bool had = m_run != -INFINITY;
        const float alpha = softmax_update<8>(x, m_run, l_run, pv);
        if (__ballot(had && alpha != 1.f)) {
#pragma unroll
            for (int ct = 0; ct < kDN / 16; ct++) o[ct] *= alpha;
        }

        // k = 32 rows: 4g+0..3 then 16+4g+0..3 (same order as pv)
        bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{bf16_pair_rne(pv[0], pv[1]), bf16_pair_rne(pv[2], pv[3]),
                          bf16_pair_rne(pv[4], pv[5]), bf16_pair_rne(pv[6], pv[7])});
        const uint16_t *v1 = ktile + (4 * g + (c >> 2)) * kKPitch + 4 * (c & 3);
        const uint16_t *v2 = v1 + 16 * kKPitch;
#pragma unroll
        for (int ct = 0; ct < kDN / 16; ct++) {
            i16x4 lo = lds_read_tr16(v1 + 16 * ct);
            i16x4 hi = lds_read_tr16(v2 + 16 * ct);
            u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
            bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
            o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[ct], 0, 0, 0);
        }
    }
    store_out(a, t, h, g, o, m_run, l_run);
}

// Decode split plan (host arithmetic only).  Head groups per workgroup: 2
// (32 heads) when H % 32 == 0, else 1.  Each (query, head block)'s list is
// cut in 16-row units and the split count with the least modelled cost is
// taken.  Cost, in units of one
// wave's compute on 32 rows for 16 heads (about 2.7 us): the larger of
//   compute  a split's rows times the share of the four consumer waves that
//            compute on each row (NG / 4), per 32 rows, and
//   gather   the bytes one workgroup pulls in (its Q rows plus its list rows
//            at the list's mean row size), per kUnitBytes,
// which overlap; plus kMergeCost for the merge of the waves sharing a head
// group and kSplitCost for splitting at all (partial store, combine
// kernel); times the waves of workgroups (one workgroup per CU: 256 run at
// once).  A workgroup resolves at most kDecMaxEntries entries and the
// combine merges at most kMaxCombineSplits splits.
void attention_plan(int n_q, int n_heads, int window, int k, bool decode, int *n_splits,
                    int *rows_per_split, int *head_groups) {
    const int entries = window + k;
    if (!decode) {
        *n_splits = 1;
        *rows_per_split = entries;
        *head_groups = 1;
        return;
    }
    constexpr int kCUs = 256, kUnit = 16;
    constexpr float kSplitCost = 3.2f, kMergeCost = 0.8f, kUnitBytes = 67500.f;
    const float row_bytes = entries > 0 ? (static_cast<float>(window) * (kD * 2) +
                                           static_cast<float>(k) * SLC_CMP_ROW_BYTES) / entries
                                        : 0.f;
    const int units = entries > 0 ? (entries + kUnit - 1) / kUnit : 1;
    const int min_splits = (entries + kDecMaxEntries - 1) / kDecMaxEntries;
    const int ng = n_heads % 32 == 0 ? 2 : 1;
    int best = -1, best_per = units;
    float best_cost = 0.f;
    const int blocks = (n_q > 0 ? n_q : 1) * (n_heads / (16 * ng));
    for (int sp = 1; sp <= kMaxCombineSplits && sp <= units; sp++) {
        const int per = (units + sp - 1) / sp;
        if (per * kUnit > kDecMaxEntries) continue;
        const int used = (units + per - 1) / per;       // splits actually formed
        if (used != sp) continue;
        const int waves = (blocks * used + kCUs - 1) / kCUs;
        const float rows = static_cast<float>(per * kUnit);
        const float compute = rows * ng / (4 * 32);
        const float gather = (16.f * ng * kD * 2 + rows * row_bytes) / kUnitBytes;
        const float cost = ((compute > gather ? compute : gather) + kMergeCost +
                            (used > 1 ? kSplitCost : 0.f)) * static_cast<float>(waves);
        if (best < 0 || cost < best_cost) {
            best = used;
            best_per = per;
            best_cost = cost;
        }
    }
    if (best < 0) {                                          // only when entries exceed the caps
        best = min_splits > 0 ? min_splits : 1;
        best_per = (units + best - 1) / best;
    }
    *rows_per_split = best_per * kUnit;
    *n_splits = (units + best_per - 1) / best_per;
    *head_groups = ng;
}

hipError_t launch_attention(const AttnArgs &a, bool decode, hipStream_t stream) {
    if (decode) {
        const int ng = a.head_groups;
        const unsigned groups = static_cast<unsigned>((a.n_q + 7) / 8);
        dim3 grid(groups * 8u * (a.n_heads / (16 * ng)) * a.n_splits);
        if (a.swa_fp8) {
            if (ng == 2) hipLaunchKernelGGL((mla_decode_kernel<2, true>), grid, dim3(512), 0, stream, a);
            else hipLaunchKernelGGL((mla_decode_kernel<1, true>), grid, dim3(512), 0, stream, a);
        } else {
            if (ng == 2) hipLaunchKernelGGL((mla_decode_kernel<2, false>), grid, dim3(512), 0, stream, a);
            else hipLaunchKernelGGL((mla_decode_kernel<1, false>), grid, dim3(512), 0, stream, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.n_splits == 1) return e;
        const int64_t threads = static_cast<int64_t>(a.n_q) * a.n_heads * (kDN / kCombCols);
        const dim3 cgrid(static_cast<unsigned>((threads + 255) / 256)), cblock(256);
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
    const int hb = (a.n_heads + 63) / 64;          // head blocks of up to 64 heads
    const int nw = a.n_heads / hb / 16;            // 16-head groups per block (uniform)
    dim3 grid(a.n_q, hb);
    if (a.swa_fp8) {
        switch (nw) {
        case 1: hipLaunchKernelGGL((mla_prefill_kernel<1, true>), grid, dim3(320), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((mla_prefill_kernel<2, true>), grid, dim3(384), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((mla_prefill_kernel<3, true>), grid, dim3(448), 0, stream, a); break;
        default: hipLaunchKernelGGL((mla_prefill_kernel<4, true>), grid, dim3(512), 0, stream, a); break;
        }
    } else {
        switch (nw) {
        case 1: hipLaunchKernelGGL((mla_prefill_kernel<1, false>), grid, dim3(320), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((mla_prefill_kernel<2, false>), grid, dim3(384), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((mla_prefill_kernel<3, false>), grid, dim3(448), 0, stream, a); break;
        default: hipLaunchKernelGGL((mla_prefill_kernel<4, false>), grid, dim3(512), 0, stream, a); break;
        }
    }
    return hipGetLastError();
}

}  // namespace slc
