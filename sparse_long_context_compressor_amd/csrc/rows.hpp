// rows.hpp -- latent rows in LDS: direct global->LDS loads of pool rows as
// stored, their LDS layouts, and the in-register dequantisation the
// decode kernels (decode.hip) apply to them.
#pragma once

#include "slc_internal.hpp"

namespace slc {

// Row pitches in LDS.  Measured on gfx950 (a microbenchmark of the kernels'
// own read patterns, eight reads in flight per wave): with a pitch of 16 B
// times 2 mod 4 units, 16-byte reads of 16 rows at one column and the
// transposing reads of 4 rows run conflict-free (5.7 and 3.8 clocks per wave
// instruction and CU); odd multiples of 16 B measured 8.1 and 5.6.
constexpr int kB16Pitch = 2 * kD + 32;          // bytes per bf16 row in LDS (1184)
constexpr int kF8Pitch = 672;                   // 512 codes | 64 bf16 rope | 8 fp32 scales
constexpr int kF8Data = SLC_CMP_ROW_BYTES;      // 640: codes + rope, then the scales
static_assert(kB16Pitch % 64 == 32 && kF8Pitch % 64 == 32, "row pitches of 2 mod 4 16-byte units");
static_assert(kF8Pitch >= kF8Data + 32, "a row's scales fit behind its codes and rope");

namespace {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Rows of skipped or padding entries are loaded from here (never written),
// so every row in LDS holds finite values.
__device__ __attribute__((aligned(256))) uint8_t kDecZeroPage[2048];

// One direct global->LDS load of 16 bytes per active lane: lane l's bytes
// land at dst + off + 16 l (dst wave-uniform); off is added to src as well.
template <int OFF>
__device__ __forceinline__ void dma16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(dst), 16, OFF, 0);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint8_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// 8 e4m3 codes (two dwords) -> 8 bf16 times a power-of-two scale, exactly.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1, float scale) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w0), scale, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w0), scale, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w1), scale, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w1), scale, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

}  // namespace

// Wait until at most n (wave-uniform, clamped to 31) of this wave's vector
// memory operations are outstanding; a larger n waits as for 31, which is
// never too short.
static __device__ __forceinline__ void wait_vmem_at_most(int n) {
#define SLC_VM_CASE(k) case k: __builtin_amdgcn_s_waitcnt(((k) & 15) | 0x70 | 0xF00 | (((k) >> 4) << 14)); break;
    switch (n < 31 ? (n < 0 ? 0 : n) : 31) {
        SLC_VM_CASE(0) SLC_VM_CASE(1) SLC_VM_CASE(2) SLC_VM_CASE(3) SLC_VM_CASE(4) SLC_VM_CASE(5)
        SLC_VM_CASE(6) SLC_VM_CASE(7) SLC_VM_CASE(8) SLC_VM_CASE(9) SLC_VM_CASE(10) SLC_VM_CASE(11)
        SLC_VM_CASE(12) SLC_VM_CASE(13) SLC_VM_CASE(14) SLC_VM_CASE(15) SLC_VM_CASE(16)
        SLC_VM_CASE(17) SLC_VM_CASE(18) SLC_VM_CASE(19) SLC_VM_CASE(20) SLC_VM_CASE(21)
        SLC_VM_CASE(22) SLC_VM_CASE(23) SLC_VM_CASE(24) SLC_VM_CASE(25) SLC_VM_CASE(26)
        SLC_VM_CASE(27) SLC_VM_CASE(28) SLC_VM_CASE(29) SLC_VM_CASE(30)
        default: __builtin_amdgcn_s_waitcnt((31 & 15) | 0x70 | 0xF00 | (1 << 14)); break;
    }
#undef SLC_VM_CASE
}

}  // namespace slc
