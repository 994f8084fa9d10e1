// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "w4a16.h"

namespace w4 {

constexpr int kGroup = 32;       // rows of K in one code block (one MFMA k step); scale groups are
                                 // kGroup << gshift rows, gshift = 0, 1, 2 (group size 32, 64, 128)
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kMaxGemvRows = 8;  // rows per GEMV task with two f16 pieces (float32 activations)
constexpr int kGemvRowsOnePiece = 16;  // rows per GEMV task with one piece (bf16 activations)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline w4a16_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Checks shared by every entry point that reads a weight descriptor.
inline w4a16_status_t check_weight(const w4a16_weight_t* w) {
  if (w == nullptr || w->qw == nullptr || w->scales == nullptr) return W4A16_ERR_INVALID_ARG;
  if (!aligned16(w->qw) || !aligned16(w->scales)) return W4A16_ERR_INVALID_ARG;
  if (w->K < 0 || w->N < 0 || w->num_experts < 1) return W4A16_ERR_INVALID_ARG;
  if (w->group_size != 32 && w->group_size != 64 && w->group_size != 128) return W4A16_ERR_UNSUPPORTED;
  if (w->K % w->group_size != 0 || w->N % 64 != 0) return W4A16_ERR_UNSUPPORTED;
  if (w->layout != W4A16_LAYOUT_CANONICAL && w->layout != W4A16_LAYOUT_GROUPED)
    return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

// log2(group size / 32) of a weight that passed check_weight.
inline int group_shift(const w4a16_weight_t* w) { return w->group_size == 128 ? 2 : (w->group_size == 64 ? 1 : 0); }

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_act(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_act<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_act<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_to_f32(p[i]);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Wave index of the calling thread as a wave-uniform value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & 63; }

}  // namespace w4
