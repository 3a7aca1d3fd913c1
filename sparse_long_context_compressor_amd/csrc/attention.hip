// attention.hip -- sparse MLA attention in absorbed (MQA) form over the
// sliding window plus the selected compressed slots, for decode (split along
// the attended list, partial softmax states merged by a second kernel) and
// prefill (one workgroup per query token).
//
// Method: "From MLA to CSA + HCA", Ch.2 (absorbed MLA: every query head
// attends one shared 576-wide latent row per entry, values are the row's
// first 512 dims); "DeepSeek-V4 attention layer types", Indexer / C4A / C128A
// (the kernel takes SWA indices together with compressed top-k indices);
// "DeepseekV4Attention" (devpress), _forward_decode / _forward_prefill.
//
// Per workgroup: 16 query heads per wave (n_heads / 16 waves), 32 attended
// entries per chunk.  Each chunk's rows are gathered through the block tables
// into an LDS tile as bf16 (compressed rows dequantised on the way: code *
// scale), then per wave:
//   S^T[32 x 16] = K[32 x 576] . Q^T[576 x 16]    (v_mfma_f32_16x16x32_bf16)
//   online softmax per head (each lane owns one head: no cross-lane rescale)
//   O^T[512 x 16] += V^T[512 x 32] . P^T[32 x 16]
// The score accumulators' lane layout already is the B-operand layout P^T
// needs (the MFMA k-order is a shared permutation of the 32 rows), and V^T
// comes from the row-major tile through ds_read_tr16_b64 (LDS transpose read),
// so the tile is written once and read twice with no transposed copy.

#include "slc_internal.hpp"

namespace slc {

namespace {

constexpr int kKPitch = kD + 8;         // bf16 per LDS row: 1168 B, spreads banks
constexpr int kUnits = kD / 8;          // 16-byte units per bf16 row (72)

typedef short lds_i16x4 __attribute__((ext_vector_type(4), address_space(3)));

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

}  // namespace

template <int NW>
__global__ __launch_bounds__(NW * 64) void mla_attn_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t ktile[kAttnChunk * kKPitch];
    __shared__ int64_t row_src[kAttnChunk];
    __shared__ int row_kind[kAttnChunk];   // 0: SWA row, 1: compressed row, -1: skipped

    constexpr int NT = NW * 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int t = blockIdx.x / a.n_splits, split = blockIdx.x % a.n_splits;
    const int seq = a.q_seq[t], p = a.q_pos[t];
    const int W = a.window;
    const int kk = a.layer_type == SLC_LAYER_SWAONLY ? 0 : a.k;
    const int E = W + kk;
    const int e_begin = split * a.chunks_per_split * kAttnChunk;
    int e_end = e_begin + a.chunks_per_split * kAttnChunk;
    e_end = e_end < E ? e_end : E;
    const int ns = kk > 0 ? a.n_slots[seq] : 0;
    const int h = 16 * w + c;

    // Q^T as the B operand: lane (g, c) holds head c, dims 8g + 32s .. +8.
    bf16x8 qb[kD / 32];
    {
        const uint16_t *qp = a.q + (static_cast<int64_t>(t) * a.n_heads + h) * kD + 8 * g;
#pragma unroll
        for (int s = 0; s < kD / 32; s++)
            qb[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(qp + 32 * s));
    }

    f32x4 o[kDN / 16];
#pragma unroll
    for (int ct = 0; ct < kDN / 16; ct++) o[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    for (int e0 = e_begin; e0 < e_end; e0 += kAttnChunk) {
        // ---- resolve the chunk's entries to physical rows ----
        if (tid < kAttnChunk) {
            int e = e0 + tid, kind = -1;
            int64_t src = -1;
            if (e < e_end) {
                if (e < W) {
                    int pos = p - W + 1 + e;
                    if (pos >= 0) src = pool_row(a.swa, seq, pos);
                    kind = src >= 0 ? 0 : -1;
                } else {
                    int s = a.cmp_idx[static_cast<int64_t>(t) * a.k + (e - W)];
                    if (s >= 0 && s < ns) src = pool_row(a.cmp, seq, s);
                    kind = src >= 0 ? 1 : -1;
                }
            }
            row_kind[tid] = kind;
            row_src[tid] = src;
        }
        __syncthreads();

        // ---- gather rows into the bf16 tile ----
        for (int u = tid; u < kAttnChunk * kUnits; u += NT) {
            int r = u / kUnits, part = u - r * kUnits;
            int kind = row_kind[r];
            int64_t src = row_src[r];
            u32x4 v = u32x4{0, 0, 0, 0};
            if (kind == 0) {
                v = *reinterpret_cast<const u32x4 *>(swa_row_ptr(a.swa, src) + 8 * part);
            } else if (kind == 1) {
                const uint8_t *rp = cmp_row_ptr(a.cmp, src);
                if (part < kDN / 8) {
                    u32x2 cw = *reinterpret_cast<const u32x2 *>(rp + 8 * part);
                    float scl = cmp_scale_ptr(a.cmp, src)[part >> 3];
                    float f[8];
                    e4m3x4_to_f32(cw[0], f[0], f[1], f[2], f[3]);
                    e4m3x4_to_f32(cw[1], f[4], f[5], f[6], f[7]);
                    v = u32x4{bf16_pair_rne(f[0] * scl, f[1] * scl),
                              bf16_pair_rne(f[2] * scl, f[3] * scl),
                              bf16_pair_rne(f[4] * scl, f[5] * scl),
                              bf16_pair_rne(f[6] * scl, f[7] * scl)};
                } else {
                    v = *reinterpret_cast<const u32x4 *>(rp + kDN + 16 * (part - kDN / 8));
                }
            }
            *reinterpret_cast<u32x4 *>(ktile + r * kKPitch + 8 * part) = v;
        }
        __syncthreads();

        // ---- S^T = K . Q^T for this wave's 16 heads ----
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

        // ---- online softmax (log2 domain); lane (g, c) holds rows 4g+i and 16+4g+i of head c ----
        float x[8];
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                int r = 16 * mt + 4 * g + i;
                x[4 * mt + i] = row_kind[r] >= 0 ? sacc[mt][i] * a.sm_scale_log2 : -INFINITY;
            }
        float cmax = x[0];
#pragma unroll
        for (int i = 1; i < 8; i++) cmax = fmaxf(cmax, x[i]);
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
        const float m_new = fmaxf(m_run, cmax);
        float pv[8], alpha = 1.f, psum = 0.f;
        if (m_new == -INFINITY) {
#pragma unroll
            for (int i = 0; i < 8; i++) pv[i] = 0.f;
        } else {
            alpha = exp2f(m_run - m_new);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                pv[i] = exp2f(x[i] - m_new);
                psum += pv[i];
            }
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int ct = 0; ct < kDN / 16; ct++) o[ct] *= alpha;

        bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{bf16_pair_rne(pv[0], pv[1]), bf16_pair_rne(pv[2], pv[3]),
                          bf16_pair_rne(pv[4], pv[5]), bf16_pair_rne(pv[6], pv[7])});

        // ---- O^T += V^T . P^T; V^T via LDS transpose reads ----
        const uint16_t *v1 = ktile + (4 * g + (c >> 2)) * kKPitch + 4 * (c & 3);
        const uint16_t *v2 = v1 + 16 * kKPitch;
#pragma unroll
        for (int ct = 0; ct < kDN / 16; ct++) {
            i16x4 lo = lds_read_tr16(v1 + 16 * ct);
            i16x4 hi = lds_read_tr16(v2 + 16 * ct);
            bf16x8 va = __builtin_bit_cast(
                bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                              __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
            o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[ct], 0, 0, 0);
        }
        __syncthreads();
    }

    // ---- epilogue: lane (g, c) holds O^T[16ct + 4g + i][head c] ----
    if (a.n_splits == 1) {
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
    } else {
        const int64_t slot = (static_cast<int64_t>(t) * a.n_splits + split) * a.n_heads + h;
        float *po = a.part_o + slot * kDN + 4 * g;
#pragma unroll
        for (int ct = 0; ct < kDN / 16; ct++) *reinterpret_cast<f32x4 *>(po + 16 * ct) = o[ct];
        if (g == 0) {
            a.part_ml[2 * slot] = m_run;
            a.part_ml[2 * slot + 1] = l_run;
        }
    }
}

// Merge the decode splits of one query: out = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
__global__ __launch_bounds__(256) void mla_combine_kernel(AttnArgs a) {
    __shared__ float sh_m[SLC_MAX_HEADS], sh_inv[SLC_MAX_HEADS];
    const int t = blockIdx.x;
    const int H = a.n_heads, S = a.n_splits;
    const int64_t base = static_cast<int64_t>(t) * S * H;
    for (int h = threadIdx.x; h < H; h += blockDim.x) {
        float M = -INFINITY;
        for (int s = 0; s < S; s++) {
            const float *ml = a.part_ml + 2 * (base + static_cast<int64_t>(s) * H + h);
            if (ml[1] > 0.f) M = fmaxf(M, ml[0]);
        }
        float L = 0.f;
        for (int s = 0; s < S; s++) {
            const float *ml = a.part_ml + 2 * (base + static_cast<int64_t>(s) * H + h);
            if (ml[1] > 0.f) L += ml[1] * exp2f(ml[0] - M);
        }
        sh_m[h] = M;
        sh_inv[h] = L > 0.f ? 1.f / L : 0.f;
        if (a.lse)
            a.lse[static_cast<int64_t>(t) * H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < H * (kDN / 4); e += blockDim.x) {
        int h = e / (kDN / 4), c4 = e - h * (kDN / 4);
        float M = sh_m[h];
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < S; s++) {
            int64_t slot = base + static_cast<int64_t>(s) * H + h;
            float l = a.part_ml[2 * slot + 1];
            if (l > 0.f) {
                float sc = exp2f(a.part_ml[2 * slot] - M);
                acc += *reinterpret_cast<const f32x4 *>(a.part_o + slot * kDN + 4 * c4) * sc;
            }
        }
        float inv = sh_inv[h];
        uint16_t *op = a.out + (static_cast<int64_t>(t) * H + h) * kDN + 4 * c4;
        *reinterpret_cast<u32x2 *>(op) = u32x2{bf16_pair_rne(acc[0] * inv, acc[1] * inv),
                                               bf16_pair_rne(acc[2] * inv, acc[3] * inv)};
    }
}

void attention_plan(int n_q, int window, int k, bool decode, int *n_splits, int *chunks_per_split) {
    int entries = window + k;
    int chunks = (entries + kAttnChunk - 1) / kAttnChunk;
    if (chunks < 1) chunks = 1;
    int target = 1;
    if (decode) {
        const int want_wgs = 512;   // about two workgroups per CU
        target = (want_wgs + n_q - 1) / (n_q > 0 ? n_q : 1);
        if (target < 1) target = 1;
    }
    int cps = (chunks + target - 1) / target;
    *chunks_per_split = cps;
    *n_splits = (chunks + cps - 1) / cps;
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t stream) {
    dim3 grid(static_cast<unsigned>(a.n_q) * a.n_splits);
    switch (a.n_heads / 16) {
    case 1: hipLaunchKernelGGL(mla_attn_kernel<1>, grid, dim3(64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(mla_attn_kernel<2>, grid, dim3(128), 0, stream, a); break;
    case 3: hipLaunchKernelGGL(mla_attn_kernel<3>, grid, dim3(192), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(mla_attn_kernel<4>, grid, dim3(256), 0, stream, a); break;
    case 5: hipLaunchKernelGGL(mla_attn_kernel<5>, grid, dim3(320), 0, stream, a); break;
    case 6: hipLaunchKernelGGL(mla_attn_kernel<6>, grid, dim3(384), 0, stream, a); break;
    case 7: hipLaunchKernelGGL(mla_attn_kernel<7>, grid, dim3(448), 0, stream, a); break;
    default: hipLaunchKernelGGL(mla_attn_kernel<8>, grid, dim3(512), 0, stream, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_splits == 1) return e;
    hipLaunchKernelGGL(mla_combine_kernel, dim3(a.n_q), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace slc
