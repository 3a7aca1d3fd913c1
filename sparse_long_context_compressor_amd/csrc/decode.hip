// decode.hip -- sparse MLA decode in absorbed (MQA) form: H query heads
// against one shared 576-wide latent row per attended entry, values from the
// row's first 512 dims ("From MLA to CSA + HCA", Ch.2), over the sliding
// window plus the compressed slots of the query's list ("DeepSeek-V4
// attention layer types", Indexer / C4A / C128A: the attention takes the SWA
// indices together with the compressed top-k indices; "DeepseekV4Attention"
// (devpress), _forward_decode).
//
// One workgroup of eight waves per (query, block of 16*HG heads, list split).
// A split takes a contiguous share of the window entries and of the
// compressed entries, and loads all of its rows into LDS at once with
// gfx950's direct global->LDS 16-byte loads, as they are stored: window rows
// as bf16 (or fp8 rows with their scales, for an fp8 window pool), compressed
// rows as e4m3 codes + bf16 rope + 8 fp32 scales.  Nothing is dequantised
// into LDS:
//   S^T = K . Q^T  v_mfma_f32_16x16x32_bf16; a lane's K operand is 16 bytes
//                  of one row that lie in one 64-dim scale block, converted
//                  exactly to bf16 with that block's scale on the way
//                  (v_cvt_scalef32_pk_bf16_fp8).  The MFMA k-order is a fixed
//                  permutation of the 576 dims, the same for K and Q.
//   O^T += V^T . P^T  the V^T operand comes straight from the row-major rows
//                  with the transposing LDS reads (ds_read_b64_tr_b8 for fp8
//                  codes, ds_read_b64_tr_b16 for bf16 rows); within one
//                  64-dim block of the output each compressed row has
//                  exactly one scale, which is folded into that row's
//                  probability (a power of two: exact).
// Lists longer than one LDS load of rows are taken in passes with an online
// softmax between them.  Splits of one query write normalised partial
// states; mla_combine_kernel merges them (attention.hip).

#include "slc_internal.hpp"
#include "rows.hpp"
#include "select.hpp"

namespace slc {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRowBytes = 132 * 1024;           // LDS for one pass's rows
constexpr int kMaxPassRows = 192;               // rows of one pass (a multiple of 32)
constexpr int kMaxKsteps = kMaxPassRows / 32;
constexpr int kOutPitch = 144;                  // bytes per head in the output stage (64 dims + pad)
// Q of one head group is staged here, later the P^T operands (both fit)
constexpr int kQpBytes = kMaxKsteps * 2 * 2 * 64 * 16;
static_assert(16 * kB16Pitch <= kQpBytes, "one head group of Q fits the P^T region");
static_assert(kWaves * 32 * kOutPitch <= kRowBytes, "the output is staged in the row region");

// The select of a workgroup's own list: 32 scores per thread (rows up to
// 16384 slots), up to 2048 prefiltered candidates; its histogram and
// candidates live in the Q / P^T region (free until the list is known).
constexpr int kSelR = 32;
constexpr int kSelMaxSlots = kThreads * kSelR;
constexpr int kSelCand = 2048;
constexpr int kMaxListShare = 512;              // list entries of one split
static_assert(hist_words<kThreads>() * 4 + 8 * kSelCand <= kQpBytes, "select scratch fits");

}  // namespace

// Grid: ceil(n_q / 8) * 8 * HB * S workgroups of 512 threads, HB = n_heads /
// (16 HG).  Blocks of one query share blockIdx % 8 (one XCD, one L2).
// F8: the window pool holds fp8 rows in the compressed-row layout.
// SEL: the workgroup selects the query's top-k list from its index scores
// itself (every workgroup of the query the same list; head block 0 writes
// its split's share of it out) before it resolves its rows.
//
// A workgroup: resolve the pass's rows, issue all their loads, then take the
// pass in stages of k-steps (32 rows): each stage waits only for its own
// rows, so its scores and value products run while later rows land.  A
// 16-row tile's scores are computed for 16 heads by a wave of that head
// group; a wave's value products cover one 64-dim output block (one scale
// per row) of every head.
template <int HG, bool F8, bool SEL>
__global__ __launch_bounds__(kThreads) void mla_decode_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t rows[kRowBytes];
    // Q staging (one head group at a time) and, after, the P^T operands
    __shared__ __attribute__((aligned(16))) uint8_t qp[kQpBytes];
    __shared__ __attribute__((aligned(16))) int32_t rid[kMaxPassRows];            // physical rows
    __shared__ float cm[kWaves][1][16];                                           // wave maxima
    __shared__ float lp[kWaves][16];                                              // wave sums
    __shared__ int32_t lst[SEL ? kMaxListShare : 1];                              // the split's list share
    __shared__ int sel_red[SEL ? 3 * kWaves : 1];
    __shared__ int sel_sh[SEL ? 8 : 1];
    f32x4 (*pfrag)[HG][2][64] = reinterpret_cast<f32x4 (*)[HG][2][64]>(qp);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c = lane & 15;

    // the prologue's kernel arguments in one round of loads
    const int32_t *q_seq_p = a.q_seq, *q_pos_p = a.q_pos, *n_slots_p = a.n_slots;
    const int32_t *cmp_idx_p = a.cmp_idx, *swa_tab = a.swa.block_table, *cmp_tab = a.cmp.block_table;
    const int swa_stride = a.swa.table_stride, cmp_stride = a.cmp.table_stride;
    const int64_t swa_nb = a.swa.n_blocks, cmp_nb = a.cmp.n_blocks;
    const int window = a.window, kk = a.k, n_q = a.n_q, S = a.n_splits;
    const int HB = a.n_heads / (16 * HG);
    __asm__ volatile("" ::"s"(q_seq_p), "s"(q_pos_p), "s"(n_slots_p), "s"(cmp_idx_p), "s"(swa_tab),
                     "s"(cmp_tab), "s"(swa_stride), "s"(cmp_stride), "s"(swa_nb), "s"(cmp_nb),
                     "s"(window), "s"(kk), "s"(n_q), "s"(S), "s"(HB));

    const int per_group = 8 * HB * S;
    const int grp = blockIdx.x / per_group, rem = blockIdx.x % per_group;
    const int t = 8 * grp + (rem & 7);
    const int hb = (rem >> 3) % HB, split = (rem >> 3) / HB;
    if (t >= n_q) return;                                         // uniform per workgroup

    // SEL: the query's score row (the select needs it before anything else),
    // 16-byte loads in the select's layout (units past the row re-read
    // its last unit; their slots lie past the visible count and are masked)
    f32x4 raw[SEL ? kSelR / 4 : 1];
    if constexpr (SEL) {
        const int msl = a.sel_max_slots;
        const float *sc = a.sel_scores + static_cast<int64_t>(t) * msl;
#pragma unroll
        for (int q = 0; q < kSelR / 4; q++) {
            const int s0 = w * 64 * kSelR + 256 * q + 4 * lane;
            raw[q] = *reinterpret_cast<const f32x4 *>(sc + (s0 < msl ? s0 : msl - 4));
        }
    }

    // ---- Q loads (they depend on nothing): the block's heads are one
    // contiguous run, 16-byte units u -> head u / 72, bytes 16 (u % 72)
    constexpr int kQUnits = 16 * HG * kD / 8;
    constexpr int kQIt = (kQUnits + kThreads - 1) / kThreads;
    u32x4 qv[kQIt];
    auto load_q = [&]() {
        const uint16_t *qsrc = a.q + (static_cast<int64_t>(t) * a.n_heads + 16 * HG * hb) * kD;
#pragma unroll
        for (int i = 0; i < kQIt; i++) {
            const int u = tid + kThreads * i;
            if (u < kQUnits) qv[i] = *reinterpret_cast<const u32x4 *>(qsrc + 8 * u);
        }
    };
    // SEL: after the select, so that its scores have the CU's loads to themselves
    if constexpr (!SEL) load_q();
    const int seq = q_seq_p[t], p = q_pos_p[t];
    const int ns = kk > 0 ? n_slots_p[seq] : 0;
    // this split's shares of the window and of the compressed list
    const int sw0 = split * a.sw_per, sw1 = min(window, sw0 + a.sw_per);
    const int cm0 = split * a.cm_per, cm1 = min(kk, cm0 + a.cm_per);
    const int n_sw = max(0, sw1 - sw0), n_cm = max(0, cm1 - cm0);
    const int sw_cap = a.sw_cap, cm_cap = a.cm_cap;
    const int passes = max(n_sw > 0 ? (n_sw + sw_cap - 1) / sw_cap : 0,
                           n_cm > 0 ? (n_cm + cm_cap - 1) / cm_cap : 0);


    // ---- pass geometry: a pass holds window rows first (padded to 32), then
    // compressed rows (padded to 32); stages: k-steps [0, KA), then the rest
    struct Geo {
        int e_sw, e_cm, nsw, ncm, nsw_pad, R, f8base, f8first, K, KA, rowsA;
    };
    auto geo = [&](int pass) {
        Geo G;
        G.e_sw = sw0 + pass * sw_cap;
        G.e_cm = cm0 + pass * cm_cap;
        G.nsw = max(0, min(sw_cap, sw1 - G.e_sw));
        G.ncm = max(0, min(cm_cap, cm1 - G.e_cm));
        G.nsw_pad = (G.nsw + 31) & ~31;
        G.R = G.nsw_pad + ((G.ncm + 31) & ~31);
        G.f8base = F8 ? 0 : G.nsw_pad * kB16Pitch;                // byte offset of the fp8 rows
        G.f8first = F8 ? 0 : G.nsw_pad;                           // first row kept as fp8
        G.K = G.R / 32;
        G.KA = G.K <= 1 ? G.K : (G.K + 1) / 2;
        G.rowsA = 32 * G.KA;
        return G;
    };
    // resolve: thread j in [lo, hi) -> physical row of pass row j (-1:
    // skipped or padding)
    auto resolve = [&](const Geo &G, int lo, int hi) {
        if (tid >= lo && tid < hi) {
            int32_t phys = -1;
            if (tid < G.nsw_pad) {
                const int pos = p - window + 1 + G.e_sw + tid;
                const int64_t lb = pos >> 6;
                if (tid < G.nsw && pos >= 0 && lb < swa_stride) {
                    const int32_t pb = swa_tab[static_cast<int64_t>(seq) * swa_stride + lb];
                    if (pb >= 0 && pb < swa_nb) phys = pb * kBR + (pos & (kBR - 1));
                }
            } else {
                const int j = tid - G.nsw_pad;
                if (j < G.ncm) {
                    const int s = SEL ? lst[G.e_cm - cm0 + j] : cmp_idx_p[static_cast<int64_t>(t) * kk + G.e_cm + j];
                    const int64_t lb = s >> 6;
                    if (s >= 0 && s < ns && lb < cmp_stride) {
                        const int32_t pb = cmp_tab[static_cast<int64_t>(seq) * cmp_stride + lb];
                        if (pb >= 0 && pb < cmp_nb) phys = pb * kBR + (s & (kBR - 1));
                    }
                }
            }
            rid[tid] = phys;
        }
    };
    // issue the loads of this wave's pass rows w + 8 i, i in [i0, i1); all
    // their ids are read first, so that no LDS access sits between the loads.
    // Returns the count of those loads that belong to the second stage.
    auto issue = [&](const Geo &G, int i0, int i1) {
        int n2 = 0;
        const int32_t my_id = w + kWaves * lane < G.R ? rid[w + kWaves * lane] : -1;
        const uint8_t *swa_b = reinterpret_cast<const uint8_t *>(a.swa.base);
        const uint8_t *cmp_b = reinterpret_cast<const uint8_t *>(a.cmp.base);
        for (int i = i0; i < i1; i++) {
            const int r = w + kWaves * i;
            const int32_t id = __builtin_amdgcn_readlane(my_id, i);
            const bool f8row = F8 || r >= G.nsw_pad;
            const bool from_swa = r < G.nsw_pad;
            if (f8row) {
                // 40 lanes: 640 bytes of codes and rope; 2 lanes: the 32 bytes of scales
                const uint8_t *blk = (from_swa ? swa_b : cmp_b) +
                                     static_cast<int64_t>(id >> 6) * SLC_CMP_BLOCK_BYTES;
                const uint8_t *src = lane < 40 ? blk + (id & 63) * SLC_CMP_ROW_BYTES + 16 * lane
                                               : blk + SLC_CMP_SCALE_OFFSET + (id & 63) * 32 + 16 * (lane - 40);
                if (id < 0) src = kDecZeroPage + 16 * lane;
                if (lane < 42) dma16<0>(src, rows + G.f8base + (r - G.f8first) * kF8Pitch);
                n2 += r >= G.rowsA ? 1 : 0;
            } else {
                const uint8_t *src = id >= 0 ? swa_b + static_cast<int64_t>(id) * (2 * kD) + 16 * lane
                                             : kDecZeroPage + 16 * lane;
                uint8_t *dst = rows + r * kB16Pitch;
                dma16<0>(src, dst);
                if (lane < 8) dma16<1024>(src, dst);
                n2 += r >= G.rowsA ? 2 : 0;
            }
        }
        return n2;
    };

    // SEL: the select, before anything that depends on the list.  (Issuing
    // pass 0's window rows ahead of it measured slower: the select then waits
    // for their table lookups, and their loads queue with the scores'.)
    if constexpr (SEL) {
        // list entries [cm0, cm1) into lst; head block 0 also writes them out
        const int msl = a.sel_max_slots;
        int n = visible_slots(p, a.sel_ratio, ns);
        n = n < msl ? n : msl;
        const bool writer = hb == 0;
        int32_t *gl = a.sel_idx + static_cast<int64_t>(t) * kk;
        if (writer && split == 0 && tid == 0) a.sel_len[t] = n < kk ? n : kk;
        if (n <= kk) {                                            // everything visible is selected
            for (int i = cm0 + tid; i < cm1; i += kThreads) {
                const int32_t v = i < n ? i : -1;
                lst[i - cm0] = v;
                if (writer) gl[i] = v;
            }
        } else {
            uint32_t *hist = reinterpret_cast<uint32_t *>(qp);
            uint32_t *cand_key = hist + hist_words<kThreads>();
            int32_t *cand_slot = reinterpret_cast<int32_t *>(cand_key + kSelCand);
            select_row<kThreads, kSelR, kSelCand>(
                raw, a.sel_scores + static_cast<int64_t>(t) * msl, n, kk,
                [&](int pos, int32_t slot) {
                    if (pos >= cm0 && pos < cm1) {
                        lst[pos - cm0] = slot;
                        if (writer) gl[pos] = slot;
                    }
                },
                hist, cand_key, cand_slot, sel_red, sel_sh);
        }
        __syncthreads();                                          // lst ready, qp free again
        // the list's stores are complete before the rows' loads go out: the
        // stage waits below count only those loads
        wait_vmem_at_most(0);
        load_q();
    }

    f32x4 o[4][HG];
#pragma unroll
    for (int dt = 0; dt < 4; dt++)
#pragma unroll
        for (int hg = 0; hg < HG; hg++) o[dt][hg] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[HG];
#pragma unroll
    for (int hg = 0; hg < HG; hg++) m_run[hg] = -INFINITY;
    float l_part = 0.f;                                           // the wave's rows' share of its head group's sums
    const float sm2 = a.sm_scale_log2;
    const int hgw = HG == 2 ? (w & 1) : 0;                         // the wave's head group (scores)
    bf16x8 qb[9][2];                                              // its Q^T operands

    for (int pass = 0; pass < passes; pass++) {
        const Geo G = geo(pass);
        const int nsw_pad = G.nsw_pad, R = G.R, f8base = G.f8base, f8first = G.f8first;
        const int K = G.K, KA = G.KA;
        resolve(G, 0, R);
        if (pass == 0) {
            // head group 0 of Q into the staging region
#pragma unroll
            for (int i = 0; i < kQIt; i++) {
                const int u = tid + kThreads * i;
                if (u < 16 * kD / 8)
                    *reinterpret_cast<u32x4 *>(qp + (u / (kD / 8)) * kB16Pitch + 16 * (u % (kD / 8))) = qv[i];
            }
        }
        __syncthreads();                                          // rid (and Q group 0) ready
        const int later = issue(G, 0, (R - w + kWaves - 1) / kWaves);   // this wave's loads of stage 2

        if (pass == 0) {
            // the wave's head group's Q^T operands, in the k-order of the K
            // operand: k-step (s, h), lane (g, c) -> head c, dims 64 s + 16 g +
            // 8 h + 0..7.  Group 0 is staged; group 1 replaces it once every
            // wave has read group 0.
#pragma unroll
            for (int hg = 0; hg < HG; hg++) {
                if (hg > 0) {
                    __syncthreads();                              // group hg-1 read
#pragma unroll
                    for (int i = 0; i < kQIt; i++) {
                        const int u = tid + kThreads * i - hg * (16 * kD / 8);
                        if (u >= 0 && u < 16 * kD / 8)
                            *reinterpret_cast<u32x4 *>(qp + (u / (kD / 8)) * kB16Pitch + 16 * (u % (kD / 8))) = qv[i];
                    }
                    __syncthreads();                              // group hg staged
                }
                if (hg == hgw) {
                    const uint8_t *qr = qp + c * kB16Pitch + 32 * g;
#pragma unroll
                    for (int s = 0; s < 9; s++)
#pragma unroll
                        for (int h = 0; h < 2; h++) qb[s][h] = ld_bf16x8(qr + 128 * s + 16 * h);
                }
            }
        }

        for (int stage = 0; stage < 2; stage++) {
            const int k0 = stage == 0 ? 0 : KA, k1 = stage == 0 ? KA : K;
            if (k0 >= k1) break;                                  // uniform
            if (stage == 0) wait_vmem_at_most(later);
            else __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();                                      // the stage's rows are in LDS

            // ---- scores: tile tau (rows 16 tau .. +15) of the stage for head
            // group hgw, by waves of that group in turn
            constexpr int kPerGroup = kWaves / HG;                // waves per head group
            constexpr int kTilesPerWave = kMaxPassRows / 32 / kPerGroup + 1;
            const int T0 = 2 * k0, T1 = 2 * k1;
            const int wq = w / HG;                                // rank within the group
            float x[kTilesPerWave][4];
            float wmax = -INFINITY;
#pragma unroll
            for (int j = 0; j < kTilesPerWave; j++) {
                const int tau = T0 + wq + kPerGroup * j;
                if (tau < T1) {                                   // wave-uniform
                    const int r0 = 16 * tau;
                    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
                    if (F8 || r0 >= nsw_pad) {
                        const uint8_t *kr = rows + f8base + (r0 - f8first + c) * kF8Pitch;
                        const f32x4 sc0 = *reinterpret_cast<const f32x4 *>(kr + kF8Data);
                        const f32x4 sc1 = *reinterpret_cast<const f32x4 *>(kr + kF8Data + 16);
                        const float scl[8] = {sc0[0], sc0[1], sc0[2], sc0[3], sc1[0], sc1[1], sc1[2], sc1[3]};
#pragma unroll
                        for (int s = 0; s < 8; s++) {
                            const u32x4 v = *reinterpret_cast<const u32x4 *>(kr + 64 * s + 16 * g);
                            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(v[0], v[1], scl[s]), qb[s][0], acc0, 0, 0, 0);
                            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(v[2], v[3], scl[s]), qb[s][1], acc1, 0, 0, 0);
                        }
                        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(kr + kDN + 32 * g), qb[8][0], acc0, 0, 0, 0);
                        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(kr + kDN + 32 * g + 16), qb[8][1], acc1, 0, 0, 0);
                    } else {
                        const uint8_t *kr = rows + (r0 + c) * kB16Pitch + 32 * g;
#pragma unroll
                        for (int s = 0; s < 9; s++) {
                            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(kr + 128 * s), qb[s][0], acc0, 0, 0, 0);
                            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ld_bf16x8(kr + 128 * s + 16), qb[s][1], acc1, 0, 0, 0);
                        }
                    }
                    const u32x4 valid = *reinterpret_cast<const u32x4 *>(rid + r0 + 4 * g);
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        x[j][i] = static_cast<int32_t>(valid[i]) >= 0 ? (acc0[i] + acc1[i]) * sm2 : -INFINITY;
                        wmax = fmaxf(wmax, x[j][i]);
                    }
                }
            }
            wmax = xor32_max(xor16_max(wmax));
            if (g == 0) cm[w][0][c] = wmax;
            __syncthreads();                                      // every wave's maxima

            // the same lazy reference update in every wave: it moves only
            // when a stage's maximum exceeds it by more than 2^8
            float alpha[HG];
#pragma unroll
            for (int hg = 0; hg < HG; hg++) {
                float mx = -INFINITY;
#pragma unroll
                for (int ww = 0; ww < kPerGroup; ww++) mx = fmaxf(mx, cm[HG * ww + hg][0][c]);
                alpha[hg] = 1.f;
                if (mx > m_run[hg] + 8.0f) {
                    alpha[hg] = m_run[hg] == -INFINITY ? 0.f : exp2f(m_run[hg] - mx);
                    m_run[hg] = mx;
                }
            }
            // probabilities of this wave's tiles -> P^T operands (k-step
            // tau/2, half tau%2: rows 4g+i, then 16+4g+i)
            {
                const float mr = m_run[hgw];
                float psum = 0.f;
#pragma unroll
                for (int j = 0; j < kTilesPerWave; j++) {
                    const int tau = T0 + wq + kPerGroup * j;
                    if (tau < T1) {
                        f32x4 pv;
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            pv[i] = mr == -INFINITY ? 0.f : exp2f(x[j][i] - mr);
                            psum += pv[i];
                        }
                        pfrag[tau >> 1][hgw][tau & 1][lane] = pv;
                    }
                }
                psum = xor32_sum(xor16_sum(psum));
                l_part = l_part * alpha[hgw] + psum;
            }
#pragma unroll
            for (int hg = 0; hg < HG; hg++)
                if (alpha[hg] != 1.f) {                           // uniform across the workgroup
#pragma unroll
                    for (int dt = 0; dt < 4; dt++) o[dt][hg] *= alpha[hg];
                }
            __syncthreads();                                      // the P^T operands

            // ---- values: wave w owns output dims 64w .. 64w+63 (scale block
            // w) for every head of the block; k-step kap covers pass rows
            // 32 kap + {4g+j, 16+4g+j}, j = 0..3, in the P^T operands' order
            for (int kap = k0; kap < k1; kap++) {
                const int rb = 32 * kap;
                const bool f8 = F8 || rb >= nsw_pad;              // uniform
                bf16x8 pb[HG];
                bf16x8 va[4];
                if (f8) {
                    // the rows' scales of block w, folded into the probabilities
                    const uint8_t *f8r = rows + f8base + (rb - f8first) * kF8Pitch;
                    float sc[8];
#pragma unroll
                    for (int j = 0; j < 8; j++) {
                        const int rr = (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
                        sc[j] = *reinterpret_cast<const float *>(f8r + rr * kF8Pitch + kF8Data + 4 * w);
                    }
#pragma unroll
                    for (int hg = 0; hg < HG; hg++) {
                        const f32x4 p0 = pfrag[kap][hg][0][lane], p1 = pfrag[kap][hg][1][lane];
                        pb[hg] = __builtin_bit_cast(
                            bf16x8, u32x4{f32x2_to_bf16x2(p0[0] * sc[0], p0[1] * sc[1]),
                                          f32x2_to_bf16x2(p0[2] * sc[2], p0[3] * sc[3]),
                                          f32x2_to_bf16x2(p1[0] * sc[4], p1[1] * sc[5]),
                                          f32x2_to_bf16x2(p1[2] * sc[6], p1[3] * sc[7])});
                    }
                    // V^T: lane (g, c) addresses row R(kap, g, c/2), bytes 8 (c%2)
                    // of each 16-dim tile of block w; it receives dim 16 dt + c of
                    // the group's 8 rows
                    const int jr = c >> 1;
                    const int rr = jr < 4 ? 4 * g + jr : 16 + 4 * g + (jr - 4);
                    const uint8_t *vr = f8r + rr * kF8Pitch + 64 * w + 8 * (c & 1);
#pragma unroll
                    for (int dt = 0; dt < 4; dt++) {
                        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (__attribute__((address_space(3))) i32x2 *)(vr + 16 * dt));
                        va[dt] = e4m3x8_to_bf16(static_cast<uint32_t>(v[0]), static_cast<uint32_t>(v[1]), 1.0f);
                    }
                } else {
#pragma unroll
                    for (int hg = 0; hg < HG; hg++) {
                        const f32x4 p0 = pfrag[kap][hg][0][lane], p1 = pfrag[kap][hg][1][lane];
                        pb[hg] = __builtin_bit_cast(
                            bf16x8, u32x4{f32x2_to_bf16x2(p0[0], p0[1]), f32x2_to_bf16x2(p0[2], p0[3]),
                                          f32x2_to_bf16x2(p1[0], p1[1]), f32x2_to_bf16x2(p1[2], p1[3])});
                    }
                    // lane (g, c) addresses rows rb + 4g + c/4 and rb + 16 + 4g + c/4,
                    // elements 4 (c%4) of each 16-dim tile; it receives element c
                    const uint8_t *v1 = rows + (rb + 4 * g + (c >> 2)) * kB16Pitch + 2 * (64 * w + 4 * (c & 3));
                    const uint8_t *v2 = v1 + 16 * kB16Pitch;
#pragma unroll
                    for (int dt = 0; dt < 4; dt++) {
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4 *)(v1 + 32 * dt));
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4 *)(v2 + 32 * dt));
                        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                        va[dt] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
                    }
                }
#pragma unroll
                for (int dt = 0; dt < 4; dt++)
#pragma unroll
                    for (int hg = 0; hg < HG; hg++)
                        o[dt][hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pb[hg], o[dt][hg], 0, 0, 0);
            }
        }
        __syncthreads();                                          // rows, rid and P^T free for the next pass
    }
    if (passes == 0) __syncthreads();                             // (nothing staged; keep the barrier count)

    // ---- the heads' sums, then this wave's 64 output dims of every head
    if (g == 0) lp[w][c] = l_part;
    __syncthreads();
    float L[HG], inv[HG];
#pragma unroll
    for (int hg = 0; hg < HG; hg++) {
        L[hg] = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves / HG; ww++) L[hg] += lp[HG * ww + hg][c];
        inv[hg] = L[hg] > 0.f ? 1.f / L[hg] : 0.f;
    }
    // O / L as bf16 through a per-wave LDS stage ([head][64 dims], pitch
    // kOutPitch), so that each store writes 128 contiguous bytes of a head
    uint8_t *stg = rows + w * (32 * kOutPitch);
#pragma unroll
    for (int hg = 0; hg < HG; hg++)
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
            *reinterpret_cast<u32x2 *>(stg + (16 * hg + c) * kOutPitch + 2 * (16 * dt + 4 * g)) =
                u32x2{f32x2_to_bf16x2(o[dt][hg][0] * inv[hg], o[dt][hg][1] * inv[hg]),
                      f32x2_to_bf16x2(o[dt][hg][2] * inv[hg], o[dt][hg][3] * inv[hg])};
    __asm__ volatile("" ::: "memory");
    const int h0 = 16 * HG * hb;
    const int64_t row0_out = S == 1 ? static_cast<int64_t>(t) * a.n_heads + h0
                                    : (static_cast<int64_t>(t) * S + split) * a.n_heads + h0;
    uint16_t *dst = (S == 1 ? a.out : a.part_o) + row0_out * kDN + 64 * w;
#pragma unroll
    for (int it = 0; it < 2 * HG; it++) {
        const int u = lane + 64 * it;                             // 16 * HG heads x 8 units
        const int hh = u >> 3, part = u & 7;
        *reinterpret_cast<u32x4 *>(dst + static_cast<int64_t>(hh) * kDN + 8 * part) =
            *reinterpret_cast<const u32x4 *>(stg + hh * kOutPitch + 16 * part);
    }
    if (w == 0 && g == 0) {
#pragma unroll
        for (int hg = 0; hg < HG; hg++) {
            const int64_t hrow = row0_out + 16 * hg + c;
            if (S == 1) {
                if (a.lse) a.lse[hrow] = L[hg] > 0.f ? (m_run[hg] + log2f(L[hg])) * kLn2 : -INFINITY;
            } else {
                a.part_ml[2 * hrow] = m_run[hg];
                a.part_ml[2 * hrow + 1] = L[hg];
            }
        }
    }
}

// Pass capacities of a decode launch (host arithmetic): each split takes
// ceil(W / S) window entries and ceil(k / S) compressed entries; a pass holds
// up to sw_cap window rows and cm_cap compressed rows (multiples of 32, at
// most kMaxPassRows in all) within kRowBytes of LDS.  Of the capacities that
// fit, those with the fewest passes are taken.
void decode_pass_caps(AttnArgs &a) {
    const int S = a.n_splits > 0 ? a.n_splits : 1;
    a.sw_per = (a.window + S - 1) / S;
    a.cm_per = (a.k + S - 1) / S;
    const int sw_row = a.swa_fp8 ? kF8Pitch : kB16Pitch;
    const int sw_max = (a.sw_per + 31) & ~31, cm_max = (a.cm_per + 31) & ~31;
    int best = -1, best_sw = 32, best_cm = 32;
    for (int sw = sw_max > 0 ? 32 : 0; sw <= sw_max; sw += 32) {
        const int left_b = kRowBytes - sw * sw_row, left_r = kMaxPassRows - sw;
        if (left_b < 0 || left_r < 0) break;
        int cm = 0;
        if (cm_max > 0) {
            cm = cm_max;
            cm = cm < (left_b / kF8Pitch) / 32 * 32 ? cm : (left_b / kF8Pitch) / 32 * 32;
            cm = cm < left_r / 32 * 32 ? cm : left_r / 32 * 32;
            if (cm < 32) continue;
        }
        const int ps = sw > 0 ? (a.sw_per + sw - 1) / sw : 0;
        const int pc = cm > 0 ? (a.cm_per + cm - 1) / cm : 0;
        const int passes = ps > pc ? ps : pc;
        if (best < 0 || passes < best) {
            best = passes;
            best_sw = sw;
            best_cm = cm;
        }
        if (sw == 0) break;
    }
    a.sw_cap = best_sw > 0 ? best_sw : 32;
    a.cm_cap = best_cm > 0 ? best_cm : 32;
}

bool decode_can_select(const AttnArgs &a0, const float *scores, int max_slots) {
    AttnArgs a = a0;
    decode_pass_caps(a);
    return scores && (reinterpret_cast<uintptr_t>(scores) & 15) == 0 && max_slots >= 4 &&
           max_slots % 4 == 0 && max_slots <= kSelMaxSlots && a.cm_per <= kMaxListShare;
}

template <bool SEL>
static void launch_decode_as(const AttnArgs &a, dim3 grid, hipStream_t stream) {
    const int hg = a.head_groups;
    if (a.swa_fp8) {
        if (hg == 2) hipLaunchKernelGGL((mla_decode_kernel<2, true, SEL>), grid, dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((mla_decode_kernel<1, true, SEL>), grid, dim3(kThreads), 0, stream, a);
    } else {
        if (hg == 2) hipLaunchKernelGGL((mla_decode_kernel<2, false, SEL>), grid, dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((mla_decode_kernel<1, false, SEL>), grid, dim3(kThreads), 0, stream, a);
    }
}

hipError_t launch_decode(const AttnArgs &a0, hipStream_t stream) {
    AttnArgs a = a0;
    decode_pass_caps(a);
    const int hg = a.head_groups;
    const unsigned groups = static_cast<unsigned>((a.n_q + 7) / 8);
    const dim3 grid(groups * 8u * (a.n_heads / (16 * hg)) * a.n_splits);
    if (a.sel_scores) launch_decode_as<true>(a, grid, stream);
    else launch_decode_as<false>(a, grid, stream);
    return hipGetLastError();
}

}  // namespace slc
