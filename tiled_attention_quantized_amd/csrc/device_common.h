// Device helpers for gfx950 (CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace taq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ _Float16 bits_to_half(uint16_t b) {
  return __builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t half_to_bits(_Float16 h) {
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ half2v u32_to_h2(uint32_t u) {
  return __builtin_bit_cast(half2v, u);
}
__device__ __forceinline__ uint32_t h2_to_u32(half2v h) {
  return __builtin_bit_cast(uint32_t, h);
}

// A 32-bit constant materialised in a VGPR.  A VALU instruction may read at
// most one scalar operand (SGPR or literal) on gfx9-family parts, so
// three-operand bit operations with two constants (v_and_or_b32, v_perm_b32)
// take one of them from a VGPR; the compiler hoists these moves out of loops.
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}

// v_perm_b32: byte i of the result is byte sel_i of the 8-byte value
// {hi = a, lo = b} (selector 0..3 -> b, 4..7 -> a, 12 -> 0x00).
__device__ __forceinline__ uint32_t perm_b32(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(a, b, sel);
}

// (x & m) | c in one v_and_or_b32 (m from a VGPR).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  return (x & vconst(m)) | c;
}

// Two unsigned bytes -> half2 (1024 + c0, 1024 + c1); exact.  `w` holds four
// bytes; hi_pair selects bytes {2,3} instead of {0,1}.
__device__ __forceinline__ uint32_t bytes_to_biased_h2(uint32_t w, bool hi_pair) {
  return perm_b32(vconst(0x64646464u), w, hi_pair ? 0x04030402u : 0x04010400u);
}

// Two nibbles at bit offsets 4k and 16 + 4k of w -> half2 of biased values,
// exact: even k gives (1024 + n, 1024 + n'), the nibbles landing in mantissa
// bits 0..3 of 1024; odd k gives (64 + n, 64 + n'), the nibbles landing in
// mantissa bits 4..7 of 64 (whose unit in the last place is 1/16), so no
// shift is needed for k = 1 and one shared shift (w8 = w >> 8) serves k = 2, 3.
__device__ __forceinline__ uint32_t nibbles_to_biased_h2(uint32_t w, uint32_t w8, int k) {
  const uint32_t x = k < 2 ? w : w8;
  return (k & 1) ? and_or(x, 0x00F000F0u, 0x54005400u) : and_or(x, 0x000F000Fu, 0x64006400u);
}
// The bias of nibbles_to_biased_h2's odd pairs is 960 below that of its even
// pairs: -(1024 + z) half2 -> -(64 + z) half2, exact for every zero byte z.
__device__ __forceinline__ uint32_t odd_nibble_negz(uint32_t nz_even) {
  return h2_to_u32(u32_to_h2(nz_even) + half2v{(_Float16)960.f, (_Float16)960.f});
}

// half2 (-(1024 + z), -(1024 + z)) for one byte z (bits 0..7 of zb).
__device__ __forceinline__ uint32_t neg_biased_zero_h2(uint32_t zb) {
  return perm_b32(vconst(0xE4E4E4E4u), zb, 0x04000400u);
}

// DPP moves inside rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// quad_perm [1,0,3,2], [2,3,0,1]; row_half_mirror; row_mirror.
constexpr int DPP_QXOR1 = 0xB1;
constexpr int DPP_QXOR2 = 0x4E;
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

// Max / sum over each row of 16 lanes; every lane gets its row's result.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<DPP_QXOR1>(x));
  x = fmaxf(x, dpp_f<DPP_QXOR2>(x));
  x = fmaxf(x, dpp_f<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp_f<DPP_MIRROR>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<DPP_QXOR1>(x);
  x += dpp_f<DPP_QXOR2>(x);
  x += dpp_f<DPP_HALF_MIRROR>(x);
  x += dpp_f<DPP_MIRROR>(x);
  return x;
}

// Read a 32-bit value from lane `src` (any lane of the wave).
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}
__device__ __forceinline__ float lane_read_f(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma16x16x32(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half8 u4_to_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }

}  // namespace taq
