// Operand helpers shared by the MFMA kernels (internal).
#pragma once

#include "common.h"

namespace w4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Exact f16 values q = nibble - 8 of one packed code word (eight consecutive
// k, nibble i at bits 4i), in the k order 0,4,1,5,2,6,3,7.  A nibble n at bits
// 0..3 of an f16 half with exponent bits 0x6400 reads as 1024 + n, so one
// packed subtraction of 1032 leaves n - 8; a nibble at bits 4..7 reads as
// 1024 + 16n and one packed fma (x / 16 - 72) leaves n - 8.  Every step is
// exact.  `magic` must hold 0x64006400 in a vector register (magic_vgpr()):
// then each mask-and-or is one v_and_or_b32, for nine vector instructions per
// word in all.
__device__ __forceinline__ half8 codes_f16(uint32_t w, uint32_t magic) {
  const uint32_t hi = w >> 8;
  const half2v sub = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const half2v sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const half2v off = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
  const half2v p0 = __builtin_bit_cast(half2v, (w & 0x000f000fu) | magic) + sub;   // k 0, 4
  const half2v p1 = __builtin_elementwise_fma(
      __builtin_bit_cast(half2v, (w & 0x00f000f0u) | magic), sixteenth, off);      // k 1, 5
  const half2v p2 = __builtin_bit_cast(half2v, (hi & 0x000f000fu) | magic) + sub;  // k 2, 6
  const half2v p3 = __builtin_elementwise_fma(
      __builtin_bit_cast(half2v, (hi & 0x00f000f0u) | magic), sixteenth, off);     // k 3, 7
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 0x64006400 in a vector register, opaque to constant folding (gfx9 VOP3
// instructions take no literal and one scalar operand, so a folded constant
// would split every v_and_or_b32 into two instructions).
__device__ __forceinline__ uint32_t magic_vgpr() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(v));
  return v;
}

// The k order in which codes_f16 lays out one block of eight.
constexpr int kCodeOrder[8] = {0, 4, 1, 5, 2, 6, 3, 7};

}  // namespace w4
