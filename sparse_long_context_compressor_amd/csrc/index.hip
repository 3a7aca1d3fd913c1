// index.hip -- lightning-indexer scores (the top-k select is in topk.hip).
//
// Method: "DeepseekV4Attention" (devpress, AMD), Indexer section:
//   I[t][s] = sum_j w[t][j] * ReLU(q[t][j] . k[s]),  H_I heads sharing one
//   key per slot, fp8 keys of 128 dims with one fp32 scale per key, or MXFP4
//   keys ("From MLA to CSA + HCA" 6.1): e2m1 values with one E8M0 scale per
//   32 dims, converted exactly to bf16 with their scale.
//
// Scores: the contraction [H_I x 128] . [128 x slots] runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).  e4m3 codes convert to bf16 exactly, and the
// bf16 MFMA accumulates at fp32 accuracy; gfx950's fp8 MFMAs accumulate the
// 128 products at a reduced internal precision (measured errors up to 1e-4 of
// sum|p|), which would break exact top-k agreement, so they are not used here.
// The contraction sits far below the bf16 ridge (the keys are the traffic),
// so the kernel stays HBM-bound.  Quantisation scales are positive, so
// ReLU(qs * ks * dot) = ks * qs * ReLU(dot) and the per-head factor w * qs is
// applied once per head, the key scale once per slot.

#include "slc_internal.hpp"

namespace slc {

namespace {

// 16 e4m3 bytes (k positions [8s, 8s+16) of the lane's share) -> two bf16x8
// MFMA operands, exactly (packed hardware conversion, unit scale).
__device__ __forceinline__ void e4m3x16_to_operands(u32x4 w, bf16x8 &s0, bf16x8 &s1) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 p[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        p[2 * i] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w[i]), 1.0f, false);
        p[2 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w[i]), 1.0f, true);
    }
    s0 = bf16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
    s1 = bf16x8{p[4][0], p[4][1], p[5][0], p[5][1], p[6][0], p[6][1], p[7][0], p[7][1]};
}

// 16 bytes of e2m1 pairs (the lane's 32 key dims, even element in the low
// nibble) times the block's E8M0 scale -> four bf16x8 MFMA operands, exactly
// (packed hardware conversion).
__device__ __forceinline__ void e2m1x32_to_operands(u32x4 w, float scale, bf16x8 (&kb)[4]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int i = 0; i < 4; i++) {
        bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 0);
        bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 1);
        bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 2);
        bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], scale, 3);
        kb[i] = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
}

// E8M0 byte -> the fp32 power of two it encodes (byte 0 -> 0: a zero block).
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
    return __uint_as_float(e << 23);
}

constexpr int kSubTiles = 16;                       // 16-key sub-tiles per wave
constexpr int kBlockSlots = 64;                     // slots per key block (one table entry)
constexpr int kRing = 4;                            // sub-tiles per load group (2 groups in flight)
constexpr int kQPitch = kDI + 16;                   // LDS bytes per staged query head
// queries per workgroup on large grids (a prefill chunk): consecutive
// queries of one sequence share every key load and key conversion
constexpr int kPrefillQT = 2;
// 64-slot blocks per such workgroup (its queries are staged once for all)
constexpr int kPrefillST = 64;
constexpr int kPrefillNS = 2;                       // spans of kPrefillST blocks per workgroup

// ReLU on the bit pattern: non-negative floats compare as non-negative ints,
// negative ones as negative ints, so one integer max does it (-0 -> +0).
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

struct KeyStage {
    u32x4 lo, hi;           // fp8: the lane's two 16-byte pieces; MXFP4: lo only
    float scale;            // fp8: the key's scale; MXFP4: the lane's block scale word
};

// Base of the zero-size buffer resource an absent block reads through.
__device__ __attribute__((aligned(256))) uint8_t kIndexZeroPage[256];   // never written

}  // namespace

// grid (n_q, ceil(max_slots / (1024 WB))), 256 WB threads: a workgroup of
// 4 WB waves scores a tile of 16 sub-tiles of WB key blocks.  WB = 2 (eight
// waves, 2048 slots) when the grid has about one workgroup per CU, as in a
// decode step: two four-wave workgroups per CU measured 3 us slower there,
// since a CU serves its loads roughly in issue order and the second
// workgroup's start waited behind the first's loads.  WB = 1 for large
// grids (prefill), where several four-wave workgroups per CU hide each
// other's latency (the eight-wave tile measured 14% slower there).
// Sub-tile j covers logical blocks s0/64 + WB j .. + WB j + WB-1: wave w
// takes slots 16*(w%4) + (0..15) of block WB j + w/4, so one (wave-uniform)
// table lookup serves each wave's sub-tile.  Lane (g = lane/16, c = lane%16)
// owns index-dim bytes [16g, 16g+16) and [64+16g, 64+16g+16) of its head
// and of its key; the MFMA k-order is the same permutation for both
// operands, so the dot product is unchanged.  F4 (MXFP4 keys): lane (g, c)
// owns dims [32g, 32g+32) instead, one 16-byte load and exactly one E8M0
// block scale, which the conversion applies.
template <int HT, int WB, bool F4>
__global__ __launch_bounds__(256 * WB) void index_score_kernel(IndexArgs a) {
    constexpr int kThreads = 256 * WB, kTile = kSubTiles * kBlockSlots * WB;
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int wq = w & 3;                                        // 16-slot quarter of a block
    const int wb = __builtin_amdgcn_readfirstlane(w >> 2);       // block within a sub-tile
    const int s0 = blockIdx.y * kTile;

    // The kernel arguments of the start-up chain in one round of loads
    // (left alone, the compiler spreads them over several dependent rounds,
    // each a full load latency before the first key is requested).
    const int32_t *q_seq_p = a.q_seq, *q_pos_p = a.q_pos, *n_slots_p = a.n_slots;
    const int32_t *table_p = a.keys.block_table;
    const int stride = a.keys.table_stride;
    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.keys.base);
    const uint8_t *zpage = kIndexZeroPage;
    const int64_t n_blocks = a.keys.n_blocks;
    __asm__ volatile("" ::"s"(q_seq_p), "s"(q_pos_p), "s"(n_slots_p), "s"(table_p), "s"(stride), "s"(kbase),
                     "s"(zpage), "s"(n_blocks));

    // The tile's 32 block-table entries first, in one load (lane j % 32 takes
    // entry j; entries past the table read entry 0 and are discarded): the
    // first key loads wait on them, and a wave's loads complete in issue
    // order.  Each sub-tile later moves its entry to a scalar register, so no
    // key load waits on a table lookup of its own.
    const int seq = q_seq_p[t];
    const int64_t table_row = static_cast<int64_t>(seq) * stride;
    int32_t my_pb;
    {
        const int64_t lb = (s0 >> 6) + (lane & (kSubTiles * WB - 1));
        const bool in = lb < stride;
        my_pb = table_p[table_row + (in ? lb : 0)];
        my_pb = in ? my_pb : -1;
    }

    int nv = 0;                                  // visible slots: read after the first key loads
    bf16x8 qa[HT][4];                            // filled after the first key loads are issued
    float hf[HT][4];

    constexpr uint32_t kKeyBytes = F4 ? kDI / 2 : kDI;
    constexpr uint32_t kBlkBytes = F4 ? SLC_KEY4_BLOCK_BYTES : SLC_KEY_BLOCK_BYTES;
    constexpr uint32_t kScaleOff = F4 ? SLC_KEY4_SCALE_OFFSET : SLC_KEY_SCALE_OFFSET;
    const uint32_t lane_off = static_cast<uint32_t>((16 * wq + c) * kKeyBytes + 16 * g);
    const uint32_t scale_off = static_cast<uint32_t>(kScaleOff + 4 * (16 * wq + c));

    // sub-tile j reads through a buffer resource on its (wave-uniform) block;
    // an absent block gets a zero-size resource, whose loads return zeros
    auto stage = [&](int j, KeyStage &st) {
        const int32_t pb = __builtin_amdgcn_readlane(my_pb, WB * j + wb);
        const bool ok = pb >= 0 && pb < n_blocks;
        const uint8_t *bp = ok ? kbase + static_cast<int64_t>(pb) * kBlkBytes : zpage;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(bp), 0, ok ? kBlkBytes : 0, kBufferWord3);
        st.lo = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, 0, 0);
        if constexpr (!F4) st.hi = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off + 64u, 0, 0);
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, scale_off, 0, 0));
        st.scale = ok ? sc : -INFINITY;
    };
    auto compute = [&](int j, const KeyStage &cur) {
        const int s = s0 + kBlockSlots * (WB * j + wb) + 16 * wq + c;
        bf16x8 kb[4];
        if constexpr (F4) {
            const uint32_t word = __builtin_bit_cast(uint32_t, cur.scale);
            e2m1x32_to_operands(cur.lo, e8m0_scale((word >> (8 * g)) & 0xffu), kb);
        } else {
            e4m3x16_to_operands(cur.lo, kb[0], kb[1]);
            e4m3x16_to_operands(cur.hi, kb[2], kb[3]);
        }
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
            for (int i = 0; i < 4; i++) part += hf[ht][i] * relu(acc[ht][i]);
        part = xor32_sum(xor16_sum(part));
        if (g == 0 && s < nv) {
            float v;
            if constexpr (F4) v = cur.scale == -INFINITY ? -INFINITY : part;   // scales applied in the dot
            else v = cur.scale == -INFINITY ? -INFINITY : part * cur.scale;
            a.scores[static_cast<int64_t>(t) * a.max_slots + s] = v;
        }
    };

    // ---- query operands and per-head factors (they depend on t only) ----
    // The query's 16*HT heads x 128 codes are one contiguous run that the
    // workgroup loads once, coalesced (per-wave operand loads would fetch it
    // four times, in half-line pieces), and stages through LDS.  With one
    // workgroup per CU (WB = 2) these loads follow the first key loads, which
    // wait only on the table; with several four-wave workgroups per CU
    // (WB = 1) they come first (measured 4% faster there), and the key
    // loads' wait on the table, issued before them, does not cover them.
    // The visible count decides the early exit after the first key loads
    // either way: those read in-range blocks or the zero page.
    constexpr int kQUnits = 16 * HT * kDI / 16;          // 16-byte units
    constexpr int kQIt = (kQUnits + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) uint8_t qlds[16 * HT * kQPitch];
    u32x4 qraw[kQIt];
    f32x4 qw[HT], qs[HT];
    auto load_query = [&]() {
        const uint8_t *qp = a.q + static_cast<int64_t>(t) * a.h_idx * kDI;
#pragma unroll
        for (int i = 0; i < kQIt; i++) {
            const int u = threadIdx.x + kThreads * i;
            if (u < kQUnits) qraw[i] = *reinterpret_cast<const u32x4 *>(qp + 16 * u);
        }
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            const int64_t o = static_cast<int64_t>(t) * a.h_idx + 16 * ht + 4 * g;   // heads 4g..4g+3
            qw[ht] = *reinterpret_cast<const f32x4 *>(a.w + o);
            qs[ht] = *reinterpret_cast<const f32x4 *>(a.q_scale + o);
        }
    };

    // two explicit buffers of kRing sub-tiles: load group q+1 while computing q
    KeyStage buf0[kRing], buf1[kRing];
    if constexpr (WB == 1) load_query();
#pragma unroll
    for (int j = 0; j < kRing; j++) stage(j, buf0[j]);
    if constexpr (WB != 1) load_query();
    nv = visible_slots(q_pos_p[t], a.ratio, n_slots_p[seq]);
    nv = nv < a.max_slots ? nv : a.max_slots;
    if (s0 >= nv) return;

#pragma unroll
    for (int i = 0; i < kQIt; i++) {
        const int u = threadIdx.x + kThreads * i;
        if (u < kQUnits)
            *reinterpret_cast<u32x4 *>(qlds + (u / (kDI / 16)) * kQPitch + 16 * (u % (kDI / 16))) = qraw[i];
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        const uint8_t *qr = qlds + (16 * ht + c) * kQPitch;
        const int q0 = F4 ? 32 * g : 16 * g, q1 = F4 ? 32 * g + 16 : 64 + 16 * g;   // the key's dims
        e4m3x16_to_operands(*reinterpret_cast<const u32x4 *>(qr + q0), qa[ht][0], qa[ht][1]);
        e4m3x16_to_operands(*reinterpret_cast<const u32x4 *>(qr + q1), qa[ht][2], qa[ht][3]);
#pragma unroll
        for (int i = 0; i < 4; i++) hf[ht][i] = qw[ht][i] * qs[ht][i];
    }
#pragma unroll
    for (int q = 0; q < kSubTiles / kRing; q++) {
        KeyStage (&cur)[kRing] = (q & 1) ? buf1 : buf0;
        KeyStage (&nxt)[kRing] = (q & 1) ? buf0 : buf1;
        if (q + 1 < kSubTiles / kRing) {
#pragma unroll
            for (int j = 0; j < kRing; j++) stage((q + 1) * kRing + j, nxt[j]);
        }
#pragma unroll
        for (int j = 0; j < kRing; j++)
            if (s0 + kBlockSlots * (WB * (q * kRing + j) + wb) < nv) compute(q * kRing + j, cur[j]);   // wave-uniform
    }
}

// Several consecutive queries per workgroup (large grids: a prefill chunk):
// four waves as in index_score_kernel<HT, 1, F4>, each taking ST 16-slot
// sub-tiles (ST 64-slot blocks per workgroup), with the workgroup's QT
// queries of one sequence sharing every key load and key conversion (their
// operands held side by side); queries of different sequences take a pass
// each.  A workgroup takes NS spans of ST blocks in turn and stages its
// queries once for all of them.
template <int HT, bool F4, int QT, int ST, int NS>
__global__ __launch_bounds__(256) void index_score_mq_kernel(IndexArgs a) {
    static_assert(ST <= 64 && (ST & (ST - 1)) == 0 && ST % 4 == 0, "one table entry per lane");
    constexpr int WB = 1;
    constexpr int RG = 2;                                        // sub-tiles per load group (registers: QT queries' operands)
    constexpr int kThreads = 256 * WB, kTile = ST * kBlockSlots * WB;
    const int t0 = blockIdx.x * QT;                              // the workgroup's queries t0 .. t0+QT-1
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int wq = w & 3;                                        // 16-slot quarter of a block
    const int wb = __builtin_amdgcn_readfirstlane(w >> 2);       // block within a sub-tile
    int s0 = blockIdx.y * NS * kTile;                            // the current span's first slot

    // The kernel arguments of the start-up chain in one round of loads
    // (left alone, the compiler spreads them over several dependent rounds,
    // each a full load latency before the first key is requested).
    const int32_t *q_seq_p = a.q_seq, *q_pos_p = a.q_pos, *n_slots_p = a.n_slots;
    const int32_t *table_p = a.keys.block_table;
    const int stride = a.keys.table_stride;
    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(a.keys.base);
    const uint8_t *zpage = kIndexZeroPage;
    const int64_t n_blocks = a.keys.n_blocks;
    const int n_q = a.n_q;
    __asm__ volatile("" ::"s"(q_seq_p), "s"(q_pos_p), "s"(n_slots_p), "s"(table_p), "s"(stride), "s"(kbase),
                     "s"(zpage), "s"(n_blocks), "s"(n_q));

    // QT > 1: queries of one sequence share every key load (one pass); else
    // (or when their sequences differ) each query takes a pass of its own
    const int nq = min(QT, n_q - t0);
    int seqs[QT];
#pragma unroll
    for (int qi = 0; qi < QT; qi++) seqs[qi] = q_seq_p[min(t0 + qi, n_q - 1)];
    bool same = true;
#pragma unroll
    for (int qi = 1; qi < QT; qi++) same = same && seqs[qi] == seqs[0];
    const int passes = same ? 1 : nq;

    // The pass's 32 block-table entries first, in one load (lane j % 32
    // takes entry j; entries past the table read entry 0 and are discarded):
    // the first key loads wait on them, and a wave's loads complete in issue
    // order.  Each sub-tile later moves its entry to a scalar register, so no
    // key load waits on a table lookup of its own.
    int32_t my_pb;
    auto lookup = [&](int seq) {
        const int64_t table_row = static_cast<int64_t>(seq) * stride;
        const int64_t lb = (s0 >> 6) + (lane & (ST * WB - 1));
        const bool in = lb < stride;
        my_pb = table_p[table_row + (in ? lb : 0)];
        my_pb = in ? my_pb : -1;
    };
    lookup(seqs[0]);

    int nv[QT];                                  // visible slots: read after the first key loads
    bf16x8 qa[QT][HT][4];                        // filled after the first key loads are issued
    float hf[QT][HT][4];

    constexpr uint32_t kKeyBytes = F4 ? kDI / 2 : kDI;
    constexpr uint32_t kBlkBytes = F4 ? SLC_KEY4_BLOCK_BYTES : SLC_KEY_BLOCK_BYTES;
    constexpr uint32_t kScaleOff = F4 ? SLC_KEY4_SCALE_OFFSET : SLC_KEY_SCALE_OFFSET;
    const uint32_t lane_off = static_cast<uint32_t>((16 * wq + c) * kKeyBytes + 16 * g);
    const uint32_t scale_off = static_cast<uint32_t>(kScaleOff + 4 * (16 * wq + c));

    // sub-tile j reads through a buffer resource on its (wave-uniform) block;
    // an absent block gets a zero-size resource, whose loads return zeros
    auto stage = [&](int j, KeyStage &st) {
        const int32_t pb = __builtin_amdgcn_readlane(my_pb, WB * j + wb);
        const bool ok = pb >= 0 && pb < n_blocks;
        const uint8_t *bp = ok ? kbase + static_cast<int64_t>(pb) * kBlkBytes : zpage;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(bp), 0, ok ? kBlkBytes : 0, kBufferWord3);
        st.lo = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, 0, 0);
        if constexpr (!F4) st.hi = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off + 64u, 0, 0);
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, scale_off, 0, 0));
        st.scale = ok ? sc : -INFINITY;
    };
    // the keys of sub-tile j against the pass's queries (every query of the
    // workgroup in a shared pass, query `pass` alone otherwise)
    auto compute = [&](int j, const KeyStage &cur, int pass) {
        const int s = s0 + kBlockSlots * (WB * j + wb) + 16 * wq + c;
        bf16x8 kb[4];
        if constexpr (F4) {
            const uint32_t word = __builtin_bit_cast(uint32_t, cur.scale);
            e2m1x32_to_operands(cur.lo, e8m0_scale((word >> (8 * g)) & 0xffu), kb);
        } else {
            e4m3x16_to_operands(cur.lo, kb[0], kb[1]);
            e4m3x16_to_operands(cur.hi, kb[2], kb[3]);
        }
        if (same && nq == QT) {                                  // uniform: every query, no branch
            // all the queries' products first, then their epilogues, in one
            // block, so that one query's epilogue can run beside the next
            // query's products
            f32x4 acc[QT][HT];
#pragma unroll
            for (int qi = 0; qi < QT; qi++)
#pragma unroll
                for (int ht = 0; ht < HT; ht++) {
                    acc[qi][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < 4; st++)
                        acc[qi][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qi][ht][st], kb[st], acc[qi][ht],
                                                                              0, 0, 0);
                }
            float part[QT];
#pragma unroll
            for (int qi = 0; qi < QT; qi++) {
                part[qi] = 0.f;
#pragma unroll
                for (int ht = 0; ht < HT; ht++)
#pragma unroll
                    for (int i = 0; i < 4; i++) part[qi] += hf[qi][ht][i] * relu(acc[qi][ht][i]);
                part[qi] = xor32_sum(xor16_sum(part[qi]));
            }
            if constexpr (QT == 2 && HT == 4 && !F4) {
                // schedule: the key conversions, the first query's 16
                // products, then each of the second query's products
                // followed by two of the first query's epilogue
                // instructions (measured 2% faster on the prefill chunk)
                __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                }
            }
#pragma unroll
            for (int qi = 0; qi < QT; qi++) {
                if (g == 0 && s < nv[qi]) {
                    float v;
                    if constexpr (F4) v = cur.scale == -INFINITY ? -INFINITY : part[qi];
                    else v = cur.scale == -INFINITY ? -INFINITY : part[qi] * cur.scale;
                    a.scores[static_cast<int64_t>(t0 + qi) * a.max_slots + s] = v;
                }
            }
            return;
        }
#pragma unroll
        for (int qi = 0; qi < QT; qi++) {
            if (!(same ? qi < nq : qi == pass)) continue;         // uniform
            f32x4 acc[HT];
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; st++)
                    acc[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qi][ht][st], kb[st], acc[ht], 0,
                                                                       0, 0);
            }
            float part = 0.f;
#pragma unroll
            for (int ht = 0; ht < HT; ht++)
#pragma unroll
                for (int i = 0; i < 4; i++) part += hf[qi][ht][i] * relu(acc[ht][i]);
            part = xor32_sum(xor16_sum(part));
            if (g == 0 && s < nv[qi]) {
                float v;
                if constexpr (F4) v = cur.scale == -INFINITY ? -INFINITY : part;   // scales applied in the dot
                else v = cur.scale == -INFINITY ? -INFINITY : part * cur.scale;
                a.scores[static_cast<int64_t>(t0 + qi) * a.max_slots + s] = v;
            }
        }
    };

    // ---- query operands and per-head factors (they depend on t only) ----
    // A query's 16*HT heads x 128 codes are one contiguous run (and the
    // workgroup's queries are consecutive) that the workgroup loads once,
    // coalesced (per-wave operand loads would fetch it four times, in
    // half-line pieces), and stages through LDS.  With one workgroup per CU
    // (WB = 2) these loads follow the first key loads, which wait only on the
    // table; with several four-wave workgroups per CU (WB = 1) they come
    // first (measured 4% faster there), and the key loads' wait on the table,
    // issued before them, does not cover them.  The visible counts decide
    // the early exit after the first key loads either way: those read
    // in-range blocks or the zero page.
    constexpr int kQUnits = QT * 16 * HT * kDI / 16;     // 16-byte units
    constexpr int kQIt = (kQUnits + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) uint8_t qlds[QT * 16 * HT * kQPitch];
    u32x4 qraw[kQIt];
    f32x4 qw[QT][HT], qs[QT][HT];
    auto load_query = [&]() {
        // units past the last query re-read the last query's (and are dropped)
        const int64_t last = static_cast<int64_t>(n_q) * a.h_idx * kDI / 16 - 1;
        const u32x4 *qp = reinterpret_cast<const u32x4 *>(a.q) + static_cast<int64_t>(t0) * a.h_idx * kDI / 16;
#pragma unroll
        for (int i = 0; i < kQIt; i++) {
            const int u = threadIdx.x + kThreads * i;
            const int64_t gu = static_cast<int64_t>(t0) * a.h_idx * kDI / 16 + u;
            if (u < kQUnits) qraw[i] = qp[gu <= last ? u : last - static_cast<int64_t>(t0) * a.h_idx * kDI / 16];
        }
#pragma unroll
        for (int qi = 0; qi < QT; qi++) {
            const int tq = min(t0 + qi, n_q - 1);
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                const int64_t o = static_cast<int64_t>(tq) * a.h_idx + 16 * ht + 4 * g;   // heads 4g..4g+3
                qw[qi][ht] = *reinterpret_cast<const f32x4 *>(a.w + o);
                qs[qi][ht] = *reinterpret_cast<const f32x4 *>(a.q_scale + o);
            }
        }
    };

    // two explicit buffers of RG sub-tiles: load group q+1 while computing q
    KeyStage buf0[RG], buf1[RG];
    if constexpr (WB == 1) load_query();
#pragma unroll
    for (int j = 0; j < RG; j++) stage(j, buf0[j]);
    if constexpr (WB != 1) load_query();
    int nv_any = 0;
#pragma unroll
    for (int qi = 0; qi < QT; qi++) {
        const int tq = min(t0 + qi, n_q - 1);
        int v = visible_slots(q_pos_p[tq], a.ratio, n_slots_p[seqs[qi]]);
        v = v < a.max_slots ? v : a.max_slots;
        nv[qi] = qi < nq ? v : 0;
        nv_any = max(nv_any, nv[qi]);
    }
    if (s0 >= nv_any) return;

#pragma unroll
    for (int i = 0; i < kQIt; i++) {
        const int u = threadIdx.x + kThreads * i;
        if (u < kQUnits)
            *reinterpret_cast<u32x4 *>(qlds + (u / (kDI / 16)) * kQPitch + 16 * (u % (kDI / 16))) = qraw[i];
    }
    __syncthreads();
#pragma unroll
    for (int qi = 0; qi < QT; qi++)
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            const uint8_t *qr = qlds + ((qi * HT + ht) * 16 + c) * kQPitch;
            const int q0 = F4 ? 32 * g : 16 * g, q1 = F4 ? 32 * g + 16 : 64 + 16 * g;   // the key's dims
            e4m3x16_to_operands(*reinterpret_cast<const u32x4 *>(qr + q0), qa[qi][ht][0], qa[qi][ht][1]);
            e4m3x16_to_operands(*reinterpret_cast<const u32x4 *>(qr + q1), qa[qi][ht][2], qa[qi][ht][3]);
#pragma unroll
            for (int i = 0; i < 4; i++) hf[qi][ht][i] = qw[qi][ht][i] * qs[qi][ht][i];
        }
    for (int span = 0; span < NS; span++) {
      if (span > 0) {                                            // the next ST blocks
        s0 += kTile;
        if (s0 >= nv_any) break;
        lookup(seqs[0]);
#pragma unroll
        for (int j = 0; j < RG; j++) stage(j, buf0[j]);
      }
      for (int pass = 0; pass < passes; pass++) {
        int nvp = nv_any;                                        // this pass's largest visible count
        if (pass > 0) {                                          // (queries of different sequences)
            lookup(seqs[pass]);
            nvp = nv[pass];
#pragma unroll
            for (int j = 0; j < RG; j++) stage(j, buf0[j]);
        } else if (!same) {
            nvp = nv[0];
        }
        // load groups alternate between the two buffers: group q + 1 loads
        // while group q is computed
        constexpr int NG = ST / RG;
        auto group = [&](int q, KeyStage (&cur)[RG], KeyStage (&nxt)[RG]) {
            if (q + 1 < NG) {
#pragma unroll
                for (int j = 0; j < RG; j++) stage((q + 1) * RG + j, nxt[j]);
            }
#pragma unroll
            for (int j = 0; j < RG; j++)
                if (s0 + kBlockSlots * (WB * (q * RG + j) + wb) < nvp) compute(q * RG + j, cur[j], pass);   // wave-uniform
        };
        for (int q = 0; q < NG; q += 2) {
            group(q, buf0, buf1);
            group(q + 1, buf1, buf0);
        }
      }
    }
}

template <int WB, bool F4>
static void launch_index(const IndexArgs &a, hipStream_t stream) {
    constexpr int tile = kSubTiles * kBlockSlots * WB;
    const dim3 grid(a.n_q, (a.max_slots + tile - 1) / tile), block(256 * WB);
    switch (a.h_idx / 16) {
    case 1: hipLaunchKernelGGL((index_score_kernel<1, WB, F4>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((index_score_kernel<2, WB, F4>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((index_score_kernel<3, WB, F4>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((index_score_kernel<4, WB, F4>), grid, block, 0, stream, a); break;
    }
}

template <bool F4>
static void launch_index_mq(const IndexArgs &a, hipStream_t stream) {
    constexpr int tile = kPrefillNS * kPrefillST * kBlockSlots;
    const dim3 grid((a.n_q + kPrefillQT - 1) / kPrefillQT, (a.max_slots + tile - 1) / tile), block(256);
    switch (a.h_idx / 16) {
    case 1: hipLaunchKernelGGL((index_score_mq_kernel<1, F4, kPrefillQT, kPrefillST, kPrefillNS>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((index_score_mq_kernel<2, F4, kPrefillQT, kPrefillST, kPrefillNS>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((index_score_mq_kernel<3, F4, kPrefillQT, kPrefillST, kPrefillNS>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((index_score_mq_kernel<4, F4, kPrefillQT, kPrefillST, kPrefillNS>), grid, block, 0, stream, a); break;
    }
}

hipError_t launch_index_scores(const IndexArgs &a, hipStream_t stream) {
    // eight-wave 2048-slot tiles while the grid stays within about two
    // workgroups per CU (256 CUs), four-wave 1024-slot tiles beyond
    constexpr int64_t kCUs = 256;
    const int64_t wide = static_cast<int64_t>(a.n_q) * ((a.max_slots + 2047) / 2048);
    if (a.key_fp4) {
        if (wide <= 2 * kCUs) launch_index<2, true>(a, stream);
        else launch_index_mq<true>(a, stream);
    } else {
        if (wide <= 2 * kCUs) launch_index<2, false>(a, stream);
        else launch_index_mq<false>(a, stream);
    }
    return hipGetLastError();
}

}  // namespace slc
