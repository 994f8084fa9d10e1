// Weight-format kernels: the quantizer, the canonical -> grouped prepack, the
// dequantize test hook and the workspace fill.
//
// Format (web page "The Weight of Precision: Building Native INT4 Quantization
// for a Custom Speculative Decoding Engine", section "The Kernel: w4a16_gemm"):
// symmetric INT4 codes, value = nibble - 8, eight nibbles per int32 along K,
// one float32 scale per 32-row group per output column (64- and 128-row
// groups are supported as well).
#include "common.h"

namespace w4 {
namespace {

__global__ void fill_zero_kernel(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                                 size_t ntail) {
  size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

// One thread per (expert, scale group, column) of `group` rows (32, 64 or
// 128).  Scale = max|w| / 7 rounded once in float32; code = round-half-even of
// the float64 quotient, clamped to [-8, 7].
__global__ void quantize_kernel(const float* __restrict__ w, int K, int N, int E, int group,
                                int32_t* __restrict__ qw, float* __restrict__ sc) {
  const int G = K / group;
  size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  size_t total = static_cast<size_t>(E) * G * N;
  if (idx >= total) return;
  const int n = static_cast<int>(idx % N);
  const size_t eg = idx / N;  // e * G + g
  const size_t e = eg / G;
  const int g = static_cast<int>(eg % G);
  const float* col = w + (e * K + static_cast<size_t>(g) * group) * N + n;
  float m = 0.0f;
  for (int r = 0; r < group; ++r) m = fmaxf(m, fabsf(col[static_cast<size_t>(r) * N]));
  const float s = __fdiv_rn(m, 7.0f);
  const double sd = static_cast<double>(s);
  int32_t* out = qw + (e * (K / 8) + static_cast<size_t>(g) * (group / 8)) * N + n;
  for (int b = 0; b < group / 8; ++b) {  // one code word per 8 rows
    uint32_t word = 0;
    for (int j = 0; j < 8; ++j) {
      int q = 0;
      if (s != 0.0f) {
        double t = rint(static_cast<double>(col[static_cast<size_t>(8 * b + j) * N]) / sd);
        t = fmin(fmax(t, -8.0), 7.0);
        q = static_cast<int>(t);
      }
      word |= static_cast<uint32_t>(q + 8) << (4 * j);
    }
    out[static_cast<size_t>(b) * N] = static_cast<int32_t>(word);
  }
  sc[eg * N + n] = s;
}

// Word index of canonical word (4g + b, n) of expert e in the GROUPED layout:
// in 64-column block j = n / 64 of group g, the 16-byte slot 16b + (n % 64) / 4
// holds word b of the four columns 4((n % 64) / 4) .. + 3, in column order.
__device__ __forceinline__ size_t grouped_word(size_t eg, int N, int n, int b) {
  const int j = n >> 6, l = (n >> 2) & 15, c = n & 3;
  return (eg * static_cast<size_t>(N / 64) + j) * 256 + 64 * b + 4 * l + c;
}

// One thread per (expert, group, column): moves the group's four canonical
// words of the column to their GROUPED slots.
__global__ void prepack_kernel(const int32_t* __restrict__ src, int K, int N, int E,
                               int32_t* __restrict__ dst) {
  const int G = K / kGroup;
  size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  size_t total = static_cast<size_t>(E) * G * N;
  if (idx >= total) return;
  const int n = static_cast<int>(idx % N);
  const size_t eg = idx / N;  // e * G + g
  const size_t e = eg / G;
  const int g = static_cast<int>(eg % G);
  const int32_t* in = src + (e * (K / 8) + static_cast<size_t>(g) * 4) * N + n;
#pragma unroll
  for (int b = 0; b < 4; ++b) dst[grouped_word(eg, N, n, b)] = in[static_cast<size_t>(b) * N];
}

// One thread per (expert, word row, column): writes float32(q * s) for the
// word's eight rows.  q * s is one IEEE float32 multiply of exact operands.
__global__ void dequantize_kernel(const int32_t* __restrict__ qw, const float* __restrict__ sc,
                                  int K, int N, int E, int group, int grouped, float* __restrict__ out) {
  const int W = K / 8;
  size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  size_t total = static_cast<size_t>(E) * W * N;
  if (idx >= total) return;
  const int n = static_cast<int>(idx % N);
  const size_t ei = idx / N;
  const size_t e = ei / W;
  const int i = static_cast<int>(ei % W);
  const int g = i >> 2;
  uint32_t word;
  if (grouped) {
    word = static_cast<uint32_t>(qw[grouped_word(e * (K / kGroup) + g, N, n, i & 3)]);
  } else {
    word = static_cast<uint32_t>(qw[ei * N + n]);
  }
  const float s = sc[(e * (K / group) + (8 * i) / group) * N + n];
  float* o = out + (e * K + static_cast<size_t>(i) * 8) * N + n;
  for (int j = 0; j < 8; ++j) {
    const float q = static_cast<float>(static_cast<int>((word >> (4 * j)) & 0xFu) - 8);
    o[static_cast<size_t>(j) * N] = __fmul_rn(q, s);
  }
}

inline unsigned grid_for(size_t total, unsigned block) {
  size_t g = (total + block - 1) / block;
  return static_cast<unsigned>(g);
}

}  // namespace
}  // namespace w4

using namespace w4;

extern "C" const char* w4a16_status_string(w4a16_status_t status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_ARG: return "invalid argument";
    case W4A16_ERR_UNSUPPORTED: return "unsupported shape, group size or layout";
    case W4A16_ERR_WORKSPACE: return "workspace too small";
    case W4A16_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

extern "C" w4a16_status_t w4a16_workspace_init(void* ws, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return W4A16_OK;
  if (ws == nullptr || !aligned16(ws)) return W4A16_ERR_INVALID_ARG;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      static_cast<uint4*>(ws), n16, static_cast<uint8_t*>(ws) + n16 * 16, ntail);
  return launch_status();
}

extern "C" w4a16_status_t w4a16_quantize_group(const float* w, int32_t K, int32_t N, int32_t E,
                                               int32_t group_size, int32_t* qw, size_t qw_bytes,
                                               float* scales, size_t scales_bytes, hipStream_t stream) {
  if (w == nullptr || qw == nullptr || scales == nullptr) return W4A16_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(qw) || !aligned16(scales)) return W4A16_ERR_INVALID_ARG;
  if (K < 0 || N < 0 || E < 0) return W4A16_ERR_INVALID_ARG;
  if (group_size != 32 && group_size != 64 && group_size != 128) return W4A16_ERR_UNSUPPORTED;
  if (K % group_size != 0) return W4A16_ERR_UNSUPPORTED;
  const size_t total = static_cast<size_t>(E) * (K / group_size) * N;
  // the outputs: E * K/8 * N code words and E * K/group_size * N scales
  if (qw_bytes < static_cast<size_t>(E) * (K / 8) * N * 4 || scales_bytes < total * 4)
    return W4A16_ERR_INVALID_ARG;
  if (total == 0) return W4A16_OK;
  quantize_kernel<<<grid_for(total, 256), 256, 0, stream>>>(w, K, N, E, group_size, qw, scales);
  return launch_status();
}

extern "C" w4a16_status_t w4a16_quantize(const float* w, int32_t K, int32_t N, int32_t E,
                                         int32_t* qw, size_t qw_bytes, float* scales, size_t scales_bytes,
                                         hipStream_t stream) {
  return w4a16_quantize_group(w, K, N, E, 32, qw, qw_bytes, scales, scales_bytes, stream);
}

extern "C" size_t w4a16_prepacked_bytes(const w4a16_weight_t* w) {
  if (check_weight(w) != W4A16_OK) return 0;
  // the GROUPED layout is a permutation of the canonical words: same size
  return static_cast<size_t>(w->num_experts) * (w->K / 8) * w->N * 4;
}

extern "C" w4a16_status_t w4a16_prepack(const w4a16_weight_t* src, int32_t* dst_qw, size_t dst_bytes,
                                        w4a16_weight_t* out, hipStream_t stream) {
  w4a16_status_t st = check_weight(src);
  if (st != W4A16_OK) return st;
  if (dst_qw == nullptr || out == nullptr || !aligned16(dst_qw)) return W4A16_ERR_INVALID_ARG;
  if (src->layout != W4A16_LAYOUT_CANONICAL) return W4A16_ERR_UNSUPPORTED;
  const size_t words = static_cast<size_t>(src->num_experts) * (src->K / 8) * src->N;
  if (dst_bytes < words * 4) return W4A16_ERR_INVALID_ARG;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(src->qw), a1 = a0 + words * 4;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(dst_qw), b1 = b0 + words * 4;
  if (words != 0 && a0 < b1 && b0 < a1) return W4A16_ERR_INVALID_ARG;
  *out = *src;
  out->qw = dst_qw;
  out->layout = W4A16_LAYOUT_GROUPED;
  const size_t total = static_cast<size_t>(src->num_experts) * (src->K / kGroup) * src->N;
  if (total == 0) return W4A16_OK;
  prepack_kernel<<<grid_for(total, 256), 256, 0, stream>>>(src->qw, src->K, src->N,
                                                           src->num_experts, dst_qw);
  return launch_status();
}

extern "C" w4a16_status_t w4a16_dequantize(const w4a16_weight_t* w, float* out, size_t out_bytes,
                                           hipStream_t stream) {
  w4a16_status_t st = check_weight(w);
  if (st != W4A16_OK) return st;
  if (out == nullptr || !aligned16(out)) return W4A16_ERR_INVALID_ARG;
  if (out_bytes < static_cast<size_t>(w->num_experts) * w->K * w->N * 4) return W4A16_ERR_INVALID_ARG;
  const size_t total = static_cast<size_t>(w->num_experts) * (w->K / 8) * w->N;
  if (total == 0) return W4A16_OK;
  dequantize_kernel<<<grid_for(total, 256), 256, 0, stream>>>(
      w->qw, w->scales, w->K, w->N, w->num_experts, w->group_size, w->layout == W4A16_LAYOUT_GROUPED, out);
  return launch_status();
}
