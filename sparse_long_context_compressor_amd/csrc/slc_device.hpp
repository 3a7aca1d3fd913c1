// slc_device.hpp -- device-side primitives shared by the gfx950 kernels:
// bf16 / OCP-e4m3 conversions, wave64 reductions, MFMA operand types and the
// paged-pool address arithmetic of the C ABI (slc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "slc.h"

namespace slc {

constexpr int kD = SLC_D_LATENT;     // 576
constexpr int kDN = SLC_D_NOPE;      // 512
constexpr int kDR = SLC_D_ROPE;      // 64
constexpr int kDI = SLC_D_INDEX;     // 128
constexpr int kBR = SLC_BLOCK_ROWS;  // 64
constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw (stride 0) buffer resource on gfx9-family targets: 32-bit
// data format, loads beyond num_records return zero.
constexpr int kBufferWord3 = 0x00020000;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN): gfx950 converts in
// hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// Two fp32 values whose low 16 mantissa bits are zero (exact bf16 values)
// packed into one dword of bf16: lo in bits 0..15, hi in 16..31.
__device__ __forceinline__ uint32_t pack_exact_bf16(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// --------------------------------------------------------------- fp8 e4m3
// gfx950 converts OCP E4M3FN in hardware (the fp8 format of this ABI).
// Four e4m3 bytes (one dword) -> four fp32, exactly.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float &a, float &b, float &c, float &d) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    a = lo[0];
    b = lo[1];
    c = hi[0];
    d = hi[1];
}

// Four e4m3 bytes -> four bf16 (exact: e4m3 has 4 significant bits) in two
// dwords, optionally multiplied by a power-of-two scale (still exact unless
// the product leaves bf16's exponent range).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w, float scale) {
    float a, b, c, d;
    e4m3x4_to_f32(w, a, b, c, d);
    u32x2 r;
    r[0] = pack_exact_bf16(a * scale, b * scale);
    r[1] = pack_exact_bf16(c * scale, d * scale);
    return r;
}

// fp32 -> e4m3 byte, round to nearest even (hardware conversion; |x| <= 448
// by construction of the caller's scale, so saturation never triggers).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false)) & 0xffu;
}

// ---------------------------------------------------------- wave64 helpers
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Combine each lane with lane ^ 16 / lane ^ 32 through gfx950's permlane
// swaps (VALU; no LDS round trip as a bpermute would take).
__device__ __forceinline__ float xor16_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide reductions and scans on DPP lane moves (VALU, no LDS): quad
// permutes and row mirrors combine within 16 lanes, the permlane swaps across
// 16 and 32.  Every lane receives the result.
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(x),
                                                             CTRL, ROW_MASK, 0xF, BOUND_ZERO));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

template <class Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t x, Op op) {
    x = op(x, dpp_u32<kDppXor1>(x, x));
    x = op(x, dpp_u32<kDppXor2>(x, x));
    x = op(x, dpp_u32<kDppHalfMirror>(x, x));
    x = op(x, dpp_u32<kDppMirror>(x, x));
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = op(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return op(r[0], r[1]);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
    return wave_allreduce_u32(x, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
    return wave_allreduce_u32(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int wave_isum(int x) {
    return static_cast<int>(wave_allreduce_u32(static_cast<uint32_t>(x),
                                               [](uint32_t a, uint32_t b) { return a + b; }));
}
// Inclusive prefix sum over lanes 0..63 (row shifts within 16 lanes, then
// the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v) {
    uint32_t x = static_cast<uint32_t>(v);
    x += dpp_u32<kDppShr1, 0xF, true>(0u, x);
    x += dpp_u32<kDppShr2, 0xF, true>(0u, x);
    x += dpp_u32<kDppShr4, 0xF, true>(0u, x);
    x += dpp_u32<kDppShr8, 0xF, true>(0u, x);
    x += dpp_u32<kDppBcast15, 0xA>(0u, x);
    x += dpp_u32<kDppBcast31, 0xC>(0u, x);
    return static_cast<int>(x);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// -------------------------------------------------------------- pool math
// Physical row of logical row `row` of sequence `seq`, or -1 if the table
// entry is absent / out of range.  Never dereferences out of bounds.
__device__ __forceinline__ int64_t pool_row(const slc_pool_t &p, int seq, int64_t row) {
    if (row < 0) return -1;
    int64_t lb = row / kBR;
    if (lb >= p.table_stride) return -1;
    int32_t pb = p.block_table[static_cast<int64_t>(seq) * p.table_stride + lb];
    if (pb < 0 || pb >= p.n_blocks) return -1;
    return static_cast<int64_t>(pb) * kBR + (row % kBR);
}

// Byte addresses inside the three pool layouts (physical row r = block*64 + i).
__device__ __forceinline__ const uint16_t *swa_row_ptr(const slc_pool_t &p, int64_t r) {
    return reinterpret_cast<const uint16_t *>(p.base) + r * kD;
}
__device__ __forceinline__ uint8_t *cmp_row_ptr(const slc_pool_t &p, int64_t r) {
    return reinterpret_cast<uint8_t *>(p.base) + (r / kBR) * SLC_CMP_BLOCK_BYTES +
           (r % kBR) * SLC_CMP_ROW_BYTES;
}
__device__ __forceinline__ float *cmp_scale_ptr(const slc_pool_t &p, int64_t r) {
    return reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(p.base) +
                                     (r / kBR) * SLC_CMP_BLOCK_BYTES + SLC_CMP_SCALE_OFFSET) +
           (r % kBR) * (kDN / 64);
}
__device__ __forceinline__ const uint8_t *key_code_ptr(const slc_pool_t &p, int64_t r) {
    return reinterpret_cast<const uint8_t *>(p.base) + (r / kBR) * SLC_KEY_BLOCK_BYTES +
           (r % kBR) * kDI;
}
__device__ __forceinline__ const float *key_scale_ptr(const slc_pool_t &p, int64_t r) {
    return reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(p.base) +
                                           (r / kBR) * SLC_KEY_BLOCK_BYTES +
                                           SLC_KEY_SCALE_OFFSET) +
           (r % kBR);
}

// Compressed slots visible to a query at position p ("From MLA to CSA + HCA",
// 5.1: position i sees slot j iff i >= r*j + r - 1), capped by the slots stored.
__device__ __forceinline__ int visible_slots(int p, int ratio, int n_slots) {
    int v = (p + 1) / ratio;
    v = v < n_slots ? v : n_slots;
    return v < 0 ? 0 : v;
}

}  // namespace slc
