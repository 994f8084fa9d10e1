// Split-K W4A16 GEMV for decode-sized row counts (vector units only).
//
// y[m][n] = sum_g s[g][n] * sum_{k in g} x[m][k] * q[k][n]   (page "The Weight
// of Precision: Building Native INT4 Quantization for a Custom Speculative
// Decoding Engine", section "The Kernel: w4a16_gemm": per-group scales on
// symmetric INT4 codes).  Each lane owns one output column and streams that
// column's 16-byte group chunks (32 codes) with one dwordx4 load per group.
// The codes are expanded to bytes holding 16*q and contracted with the
// activation's fixed-point pieces by v_dot4_i32_i8; the pieces are
// wave-uniform and live in scalar registers.  The per-group integer sums are
// exact; each becomes float32 once and is scaled by s * factor.
#include "gemv.h"

namespace w4 {
namespace {

// ------------------------------------------------------------ fixed-point pieces

template <int P>
__device__ __forceinline__ int piece_shift(float amax) {
  if (!(amax > 0.0f)) return 0;
  constexpr int L = 8 * P - 2;  // |X| <= 2^L
  int sh = (L - 1) - ilogbf(amax);
  return sh > 120 ? 120 : sh;
}

template <int P>
__device__ __forceinline__ void split_pieces(float v, int sh, int pc[P]) {
  int X = static_cast<int>(rintf(ldexpf(v, sh)));
  if (P == 3) {
    const int p2 = static_cast<int8_t>(X & 0xff);
    const int t = (X - p2) >> 8;
    const int p1 = static_cast<int8_t>(t & 0xff);
    pc[0] = (t - p1) >> 8;
    pc[1] = p1;
    pc[P - 1] = p2;
  } else {
    const int p1 = static_cast<int8_t>(X & 0xff);
    pc[0] = (X - p1) >> 8;
    pc[P - 1] = p1;
  }
}

// Byte offset of (piece p, element c) inside one (row, group) block.
__device__ __forceinline__ int piece_byte(int p, int c) {
  const int j = c >> 3, b = c & 7;
  return (((p * 4 + j) * 2 + (b & 1)) << 2) + (b >> 1);
}

// One thread per (position, group).
template <typename XT, int P>
__global__ void prep_pieces_kernel(const XT* __restrict__ x, int R, int K,
                                   const int* __restrict__ sorted_pairs, int top_k,
                                   int32_t* __restrict__ xq, float* __restrict__ xf) {
  const int G = K / kGroup;
  const size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (idx >= static_cast<size_t>(R) * G) return;
  const int pos = static_cast<int>(idx % R);
  const int g = static_cast<int>(idx / R);
  long row = pos;
  if (sorted_pairs != nullptr) {
    const int pr = sorted_pairs[pos];
    row = pr < 0 ? -1 : pr / top_k;
  }
  float v[kGroup];
  float amax = 0.0f;
  const XT* src = x + (row < 0 ? 0 : row) * K + static_cast<size_t>(g) * kGroup;
#pragma unroll
  for (int c = 0; c < kGroup; ++c) {
    v[c] = row < 0 ? 0.0f : load_act(src, c);
    amax = fmaxf(amax, fabsf(v[c]));
  }
  const int sh = piece_shift<P>(amax);
  uint32_t dw[8 * P];
#pragma unroll
  for (int i = 0; i < 8 * P; ++i) dw[i] = 0;
#pragma unroll
  for (int c = 0; c < kGroup; ++c) {
    int pc[P];
    split_pieces<P>(v[c], sh, pc);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int byte = piece_byte(p, c);
      dw[byte >> 2] |= (static_cast<uint32_t>(pc[p]) & 0xffu) << (8 * (byte & 3));
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(xq + idx * (8 * P));  // idx == g * R + pos
#pragma unroll
  for (int i = 0; i < 2 * P; ++i) {
    u32x4 t = {dw[4 * i], dw[4 * i + 1], dw[4 * i + 2], dw[4 * i + 3]};
    dst[i] = t;
  }
  xf[idx] = amax > 0.0f ? ldexpf(1.0f, -sh - 4) : 0.0f;
}

// ------------------------------------------------------------ the GEMV core

// Integer dot of one row's pieces with one group's byte-expanded codes.
template <int P>
__device__ __forceinline__ float group_dot(const int32_t* __restrict__ xp, const int32_t we[4],
                                           const int32_t wo[4]) {
  int a = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a = __builtin_amdgcn_sdot4(xp[j * 2 + 0], we[j], a, false);
    a = __builtin_amdgcn_sdot4(xp[j * 2 + 1], wo[j], a, false);
  }
  a *= 256;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a = __builtin_amdgcn_sdot4(xp[8 + j * 2 + 0], we[j], a, false);
    a = __builtin_amdgcn_sdot4(xp[8 + j * 2 + 1], wo[j], a, false);
  }
  if (P == 2) return static_cast<float>(a);
  int b = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b = __builtin_amdgcn_sdot4(xp[16 + j * 2 + 0], we[j], b, false);
    b = __builtin_amdgcn_sdot4(xp[16 + j * 2 + 1], wo[j], b, false);
  }
  return fmaf(static_cast<float>(a), 256.0f, static_cast<float>(b));
}

__device__ __forceinline__ void expand_codes(const u32x4 w, int32_t we[4], int32_t wo[4]) {
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // byte b of we: 16*(nibble 2b - 8); byte b of wo: 16*(nibble 2b+1 - 8)
    we[j] = static_cast<int32_t>(((v[j] << 4) & 0xf0f0f0f0u) ^ 0x80808080u);
    wo[j] = static_cast<int32_t>((v[j] & 0xf0f0f0f0u) ^ 0x80808080u);
  }
}

constexpr int kUnroll = 4;

template <int P, int NR>
__device__ __forceinline__ void gemv_rows(const u32x4* __restrict__ wq, const float* __restrict__ ws,
                                          size_t gstride, const int32_t* __restrict__ xq,
                                          const float* __restrict__ xf, size_t R, int g_lo,
                                          int g_hi, float acc[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0f;
  int g = g_lo;
  for (; g + kUnroll <= g_hi; g += kUnroll) {
    u32x4 w[kUnroll];
    float s[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      w[u] = __builtin_nontemporal_load(wq + static_cast<size_t>(g + u) * gstride);
      s[u] = __builtin_nontemporal_load(ws + static_cast<size_t>(g + u) * gstride);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int32_t we[4], wo[4];
      expand_codes(w[u], we, wo);
      const int32_t* xg = xq + static_cast<size_t>(g + u) * R * (8 * P);
      const float* fg = xf + static_cast<size_t>(g + u) * R;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float F = group_dot<P>(xg + r * (8 * P), we, wo);
        acc[r] = fmaf(s[u] * fg[r], F, acc[r]);
      }
    }
  }
  for (; g < g_hi; ++g) {
    const u32x4 w = __builtin_nontemporal_load(wq + static_cast<size_t>(g) * gstride);
    const float s = __builtin_nontemporal_load(ws + static_cast<size_t>(g) * gstride);
    int32_t we[4], wo[4];
    expand_codes(w, we, wo);
    const int32_t* xg = xq + static_cast<size_t>(g) * R * (8 * P);
    const float* fg = xf + static_cast<size_t>(g) * R;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float F = group_dot<P>(xg + r * (8 * P), we, wo);
      acc[r] = fmaf(s * fg[r], F, acc[r]);
    }
  }
}

template <int P, int NR>
__device__ __forceinline__ void run_rows(const GemvArgs& a, const u32x4* wq, const float* ws,
                                         int pos0, int g_lo, int g_hi,
                                         float red[][kMaxGemvRows][64], int wv, int lane) {
  float acc[NR];
  gemv_rows<P, NR>(wq, ws, a.N, a.xq + static_cast<size_t>(pos0) * (8 * P), a.xf + pos0,
                   static_cast<size_t>(a.R), g_lo, g_hi, acc);
#pragma unroll
  for (int r = 0; r < NR; ++r) red[wv][r][lane] = acc[r];
}

template <int P>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const GemvArgs a) {
  __shared__ float red[kGemvThreads / kWave][kMaxGemvRows][64];
  __shared__ int sh_last;

  const int task = blockIdx.x;
  const int split = task % a.S;
  const int rest = task / a.S;
  const int tile = rest % a.tiles;
  const int item = rest / a.tiles;

  int expert = 0, pos0, nrows;
  if (a.dense_rows > 0) {
    pos0 = item * kMaxGemvRows;
    nrows = min(kMaxGemvRows, a.dense_rows - pos0);
  } else {
    if (item >= *a.n_items) return;
    const int4 it = a.items[item];
    expert = it.x;
    pos0 = it.y;
    nrows = it.z;
  }

  const int wv = wave_id();
  const int lane = lane_id();
  int mat = 0, col;
  if (a.mode == 1) {
    mat = lane >> 5;
    col = tile * 32 + (lane & 31);
  } else {
    col = tile * 64 + lane;
  }
  const size_t ebase = static_cast<size_t>(expert) * a.expert_stride;
  const u32x4* wq = (mat ? a.qw1 : a.qw0) + ebase + col;
  const float* ws = (mat ? a.sc1 : a.sc0) + ebase + col;

  const int sg_lo = split * a.gps;
  const int sg_hi = min(a.G, sg_lo + a.gps);
  const int nw = kGemvThreads / kWave;
  const int span = (sg_hi - sg_lo + nw - 1) / nw;
  const int g_lo = min(sg_hi, sg_lo + wv * span);
  const int g_hi = min(sg_hi, g_lo + span);

  switch (nrows) {
    case 1: run_rows<P, 1>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
    case 2: run_rows<P, 2>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
    case 3: run_rows<P, 3>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
    case 4: run_rows<P, 4>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
    case 5: run_rows<P, 5>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
    case 6: run_rows<P, 6>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
    case 7: run_rows<P, 7>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
    default: run_rows<P, 8>(a, wq, ws, pos0, g_lo, g_hi, red, wv, lane); break;
  }
  __syncthreads();

  // fixed-order reduction over the four waves, then over the K splits
  float v[kMaxGemvRows];
  if (wv == 0) {
#pragma unroll
    for (int r = 0; r < kMaxGemvRows; ++r) {
      if (r < nrows) v[r] = ((red[0][r][lane] + red[1][r][lane]) + red[2][r][lane]) + red[3][r][lane];
    }
  }
  if (a.S > 1) {
    const size_t ct = static_cast<size_t>(item) * a.tiles + tile;
    float* base = a.partials + ct * a.S * kPartialTileFloats;
    if (wv == 0) {
      for (int r = 0; r < nrows; ++r) base[split * kPartialTileFloats + r * 64 + lane] = v[r];
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = atomicAdd(&a.counters[ct], 1);
      sh_last = (prev == a.S - 1);
    }
    __syncthreads();
    if (!sh_last) return;
    __threadfence();
    if (wv == 0) {
      for (int r = 0; r < nrows; ++r) {
        float t = 0.0f;
        for (int s = 0; s < a.S; ++s) t += base[s * kPartialTileFloats + r * 64 + lane];
        v[r] = t;
      }
    }
    if (threadIdx.x == 0) a.counters[ct] = 0;
  }
  if (wv != 0) return;

  if (a.mode == 0) {
    for (int r = 0; r < nrows; ++r)
      a.out[static_cast<size_t>(pos0 + r) * a.N + col] = v[r];
    return;
  }

  // SwiGLU epilogue: lanes 0..31 hold gate, 32..63 up, for columns tile*32 + c.
  // The 32 columns are one scale group of the down projection's input, so the
  // pieces of h are formed here directly.
  const int c = lane & 31;
  for (int r = 0; r < nrows; ++r) {
    const float up = __shfl_down(v[r], 32);
    const float h = silu(v[r]) * up;
    float amax = lane < 32 ? fabsf(h) : 0.0f;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const size_t prow = static_cast<size_t>(pos0 + r);
    if (lane < 32) {
      const int sh = piece_shift<P>(amax);
      int pc[P];
      split_pieces<P>(h, sh, pc);
      uint8_t* blk = reinterpret_cast<uint8_t*>(a.hq + (static_cast<size_t>(tile) * a.R + prow) * (8 * P));
#pragma unroll
      for (int p = 0; p < P; ++p) blk[piece_byte(p, c)] = static_cast<uint8_t>(pc[p] & 0xff);
      if (c == 0) a.hf[static_cast<size_t>(tile) * a.R + prow] = amax > 0.0f ? ldexpf(1.0f, -sh - 4) : 0.0f;
      if (a.h_raw != nullptr) {
        const size_t hi = prow * a.N + tile * 32 + c;
        if (a.h_bf16)
          static_cast<uint16_t*>(a.h_raw)[hi] = f32_to_bf16(h);
        else
          static_cast<float*>(a.h_raw)[hi] = h;
      }
    }
  }
}

}  // namespace

int gemv_splits(size_t tasks, int G) {
  // aim for about 1024 workgroups (4 per CU) while keeping >= 8 groups per wave
  const size_t target = 1024;
  int S = static_cast<int>((target + tasks - 1) / tasks);
  const int max_s = G / (8 * (kGemvThreads / kWave));
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  return S;
}

w4a16_status_t launch_prep_pieces(const void* x, w4a16_dtype_t xt, int R, int K, int P,
                                  const int* sorted_pairs, int top_k, int32_t* xq, float* xf,
                                  hipStream_t stream) {
  const size_t total = static_cast<size_t>(R) * (K / kGroup);
  if (total == 0) return W4A16_OK;
  const unsigned grid = static_cast<unsigned>((total + 127) / 128);
  if (xt == W4A16_F32 && P == 3)
    prep_pieces_kernel<float, 3><<<grid, 128, 0, stream>>>(static_cast<const float*>(x), R, K,
                                                           sorted_pairs, top_k, xq, xf);
  else if (xt == W4A16_BF16 && P == 2)
    prep_pieces_kernel<uint16_t, 2><<<grid, 128, 0, stream>>>(static_cast<const uint16_t*>(x), R, K,
                                                              sorted_pairs, top_k, xq, xf);
  else if (xt == W4A16_F32 && P == 2)
    prep_pieces_kernel<float, 2><<<grid, 128, 0, stream>>>(static_cast<const float*>(x), R, K,
                                                           sorted_pairs, top_k, xq, xf);
  else
    prep_pieces_kernel<uint16_t, 3><<<grid, 128, 0, stream>>>(static_cast<const uint16_t*>(x), R, K,
                                                              sorted_pairs, top_k, xq, xf);
  return launch_status();
}

w4a16_status_t launch_gemv(const GemvArgs& a, int P, size_t num_tasks, hipStream_t stream) {
  if (num_tasks == 0) return W4A16_OK;
  if (num_tasks > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  const unsigned grid = static_cast<unsigned>(num_tasks);
  if (P == 3)
    gemv_kernel<3><<<grid, kGemvThreads, 0, stream>>>(a);
  else
    gemv_kernel<2><<<grid, kGemvThreads, 0, stream>>>(a);
  return launch_status();
}

}  // namespace w4
