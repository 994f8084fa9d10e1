// Split-K W4A16 GEMV for decode-sized row counts (vector units only).
//
// y[m][n] = sum_g s[g][n] * sum_{k in g} x[m][k] * q[k][n]   (page "The Weight
// of Precision: Building Native INT4 Quantization for a Custom Speculative
// Decoding Engine", section "The Kernel: w4a16_gemm": per-group scales on
// symmetric INT4 codes).
//
// Each lane owns SUB output columns (64 apart, so one wave load reads 1 KiB of
// contiguous 16-byte group chunks) and streams one chunk (32 codes) per group
// and column.  The codes need one XOR to become signed nibbles; activations
// are signed 4-bit digits of per-group fixed point (gemv.h), staged by each
// wave in its own LDS window and read back as uniform vectors.  v_dot8_i32_i4
// contracts eight codes with eight digits, Horner steps by 16 join the
// digits, and each group's exact integer sum becomes float32 once and is
// scaled by s * 2^-sh.
#include "gemv.h"

namespace w4 {
namespace {

constexpr int kWin = 8;  // groups per staging window of one wave

// Largest sh with amax * 2^sh <= 3 * 2^(4D-3).
template <int D>
__device__ __forceinline__ int digit_shift(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = ilogbf(amax);
  const float m = ldexpf(amax, -e);  // [1, 2)
  const int sh = (4 * D - 2 - e) - (m > 1.5f ? 1 : 0);
  return sh > 120 ? 120 : sh;
}

// Biased fixed point of v: the low 4D bits of the result are X + B with
// X = round(v * 2^sh) and B = 8 * (16^D - 1) / 15, so hex digit d (from the top)
// of X + B is the balanced digit d of X plus 8.  One FMA: adding 2^23 + B to the
// exact product v * 2^sh leaves the rounded integer in the float's mantissa
// bits (|X| + B < 2^23).
template <int D>
__device__ __forceinline__ uint32_t biased_fixed(float v, float scale) {
  constexpr float kMagic = 8388608.0f + static_cast<float>(8 * ((1 << (4 * D)) - 1) / 15);
  return __float_as_uint(fmaf(v, scale, kMagic));
}

// Balanced digit d (most significant first) of a biased_fixed value, as a
// two's-complement nibble in bits 0..3.
template <int D>
__device__ __forceinline__ uint32_t digit_nibble(uint32_t xb, int d) {
  return ((xb >> (4 * (D - 1 - d))) & 15u) ^ 8u;
}

template <int D>
struct WaveWindow {
  int32_t dig[kWin][kMaxGemvRows][4 * D];
  float fac[kWin][kMaxGemvRows];
};

template <int D, int SUB>
union GemvLds {
  WaveWindow<D> win[kGemvThreads / kWave];
  float red[kGemvThreads / kWave][kMaxGemvRows][64 * SUB];
};

template <typename XT>
__device__ __forceinline__ float act(const void* x, size_t i) {
  return load_act(static_cast<const XT*>(x), i);
}

// Lane (gi, r) = (lane >> 3, lane & 7) fills item (group gw + gi, row r) of the
// wave's window.
template <int D, int IN>
__device__ __forceinline__ void stage_window(const GemvArgs& a, WaveWindow<D>& w, int gw, int nw,
                                             int pos0, int nrows, int lane) {
  const int gi = lane >> 3, r = lane & 7;
  if (gi >= nw || r >= nrows) return;
  const int g = gw + gi;
  const int pos = pos0 + r;
  if (IN == kInDigits) {
    const int32_t* src = a.xq + (static_cast<size_t>(g) * a.R + pos) * (4 * D);
#pragma unroll
    for (int i = 0; i < 4 * D; ++i) w.dig[gi][r][i] = src[i];
    w.fac[gi][r] = a.xf[static_cast<size_t>(g) * a.R + pos];
    return;
  }
  long row = pos;
  if (a.gather != nullptr) {
    const int pr = a.gather[pos];
    row = pr < 0 ? -1 : pr / a.top_k;
  }
  // two passes over the group's 32 activations (the second hits the cache):
  // the largest magnitude first, then the digits, eight elements at a time
  const size_t base = static_cast<size_t>(row < 0 ? 0 : row) * a.K + static_cast<size_t>(g) * kGroup;
  float amax = 0.0f;
  if (row >= 0) {
#pragma unroll
    for (int c = 0; c < kGroup; ++c)
      amax = fmaxf(amax, fabsf(IN == kInF32 ? act<float>(a.x, base + c) : act<uint16_t>(a.x, base + c)));
  }
  const int sh = digit_shift<D>(amax);
  const float scale = row < 0 ? 0.0f : ldexpf(1.0f, sh);
  uint32_t dw[4 * D];
#pragma unroll
  for (int i = 0; i < 4 * D; ++i) dw[i] = 0;
#pragma unroll
  for (int c = 0; c < kGroup; ++c) {
    const float xv = row < 0 ? 0.0f : (IN == kInF32 ? act<float>(a.x, base + c) : act<uint16_t>(a.x, base + c));
    const uint32_t xb = biased_fixed<D>(xv, scale);
#pragma unroll
    for (int d = 0; d < D; ++d)
      dw[d * 4 + (c >> 3)] |= ((xb >> (4 * (D - 1 - d))) & 15u) << (4 * (c & 7));
  }
#pragma unroll
  for (int i = 0; i < 4 * D; ++i) w.dig[gi][r][i] = static_cast<int32_t>(dw[i] ^ 0x88888888u);
  w.fac[gi][r] = amax > 0.0f ? ldexpf(1.0f, -sh) : 0.0f;
}

template <int SUB>
__device__ __forceinline__ void load_group(const u32x4* __restrict__ wq, const float* __restrict__ ws,
                                           size_t gstride, int cstride, int g, u32x4 w[SUB],
                                           float s[SUB]) {
#pragma unroll
  for (int j = 0; j < SUB; ++j) {
    w[j] = __builtin_nontemporal_load(wq + static_cast<size_t>(g) * gstride + cstride * j);
    s[j] = __builtin_nontemporal_load(ws + static_cast<size_t>(g) * gstride + cstride * j);
  }
}

// One wave: groups [g_lo, g_hi) of its columns, NR rows from position pos0.
template <int D, int NR, int SUB, int IN>
__device__ __forceinline__ void wave_gemv(const GemvArgs& a, const u32x4* wq, const float* ws,
                                          int cstride, int pos0, int g_lo, int g_hi,
                                          WaveWindow<D>& win, int lane, float acc[SUB][NR]) {
#pragma unroll
  for (int j = 0; j < SUB; ++j)
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[j][r] = 0.0f;
  const size_t gstride = static_cast<size_t>(a.N);
  for (int gw = g_lo; gw < g_hi; gw += kWin) {
    const int nw = min(kWin, g_hi - gw);
    u32x4 wc[SUB];
    float sc[SUB];
    load_group<SUB>(wq, ws, gstride, cstride, gw, wc, sc);
    stage_window<D, IN>(a, win, gw, nw, pos0, NR, lane);
    __builtin_amdgcn_wave_barrier();
    for (int gi = 0; gi < nw; ++gi) {
      u32x4 wn[SUB];
      float sn[SUB];
      load_group<SUB>(wq, ws, gstride, cstride, gw + min(gi + 1, nw - 1), wn, sn);
      int32_t q[SUB][4];
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        q[j][0] = static_cast<int32_t>(wc[j].x ^ 0x88888888u);
        q[j][1] = static_cast<int32_t>(wc[j].y ^ 0x88888888u);
        q[j][2] = static_cast<int32_t>(wc[j].z ^ 0x88888888u);
        q[j][3] = static_cast<int32_t>(wc[j].w ^ 0x88888888u);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int32_t* dp = win.dig[gi][r];
        int32_t dg[4 * D];
#pragma unroll
        for (int i = 0; i < 4 * D; ++i) dg[i] = dp[i];
        const float f = win.fac[gi][r];
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
          int t = 0;
#pragma unroll
          for (int d = 0; d < D; ++d) {
            t *= 16;
#pragma unroll
            for (int i = 0; i < 4; ++i) t = __builtin_amdgcn_sdot8(dg[d * 4 + i], q[j][i], t, false);
          }
          acc[j][r] = fmaf(sc[j] * f, static_cast<float>(t), acc[j][r]);
        }
      }
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        wc[j] = wn[j];
        sc[j] = sn[j];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int D, int NR, int SUB, int IN>
__device__ __forceinline__ void run_rows(const GemvArgs& a, const u32x4* wq, const float* ws,
                                         int cstride, int pos0, int g_lo, int g_hi,
                                         GemvLds<D, SUB>& lds, int wv, int lane) {
  float acc[SUB][NR];
  wave_gemv<D, NR, SUB, IN>(a, wq, ws, cstride, pos0, g_lo, g_hi, lds.win[wv], lane, acc);
  __syncthreads();  // every wave is done with its window before the buffer is reused
#pragma unroll
  for (int j = 0; j < SUB; ++j)
#pragma unroll
    for (int r = 0; r < NR; ++r) lds.red[wv][r][64 * j + lane] = acc[j][r];
}

template <int D, int SUB, int IN>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(W4_GEMV_WAVES_PER_EU)))
void gemv_kernel(const GemvArgs a) {
  __shared__ GemvLds<D, SUB> lds;
  __shared__ int last;
  constexpr int TW = 64 * SUB;  // values per row of one tile

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
  // plain tiles: 64*SUB consecutive columns, sub-column j at +64j; SwiGLU tiles:
  // 32*SUB gate columns (lanes 0..31) and the same up columns (lanes 32..63),
  // sub-column j at +32j
  int mat = 0, col0;
  if (a.mode == 1) {
    mat = lane >> 5;
    col0 = tile * 32 * SUB + (lane & 31);
  } else {
    col0 = tile * TW + lane;
  }
  const int cstride = a.mode == 1 ? 32 : 64;
  const size_t ebase = static_cast<size_t>(expert) * a.expert_stride;
  const u32x4* wq = (mat ? a.qw1 : a.qw0) + ebase + col0;
  const float* wsc = (mat ? a.sc1 : a.sc0) + ebase + col0;

  const int sg_lo = split * a.gps;
  const int sg_hi = min(a.G, sg_lo + a.gps);
  const int nw = kGemvThreads / kWave;
  const int span = (sg_hi - sg_lo + nw - 1) / nw;
  const int g_lo = min(sg_hi, sg_lo + wv * span);
  const int g_hi = min(sg_hi, g_lo + span);

  switch (nrows) {
#define W4_CASE(n) \
  case n: run_rows<D, n, SUB, IN>(a, wq, wsc, cstride, pos0, g_lo, g_hi, lds, wv, lane); break;
    W4_CASE(1) W4_CASE(2) W4_CASE(3) W4_CASE(4) W4_CASE(5) W4_CASE(6) W4_CASE(7)
    default: run_rows<D, 8, SUB, IN>(a, wq, wsc, cstride, pos0, g_lo, g_hi, lds, wv, lane); break;
#undef W4_CASE
  }
  __syncthreads();

  // Fixed-order reduction over the four waves, then over the K splits.  Thread
  // t owns elements e = t + 256i of the tile [nrows][TW].
  constexpr int kEl = kMaxGemvRows * TW / kGemvThreads;  // elements per thread (upper bound)
  float* tilev = &lds.red[0][0][0];  // reduced tile, row stride TW
  float v[kEl];
#pragma unroll
  for (int i = 0; i < kEl; ++i) {
    const int e = static_cast<int>(threadIdx.x) + kGemvThreads * i;
    const int r = e / TW, cc = e % TW;
    v[i] = r < nrows ? ((lds.red[0][r][cc] + lds.red[1][r][cc]) + lds.red[2][r][cc]) + lds.red[3][r][cc]
                     : 0.0f;
  }
  if (a.S > 1) {
    // Partials are written through to the device coherence point (agent-scope
    // stores), the arrival counter is an agent-scope atomic, and the last
    // workgroup of the tile reads every partial back with agent-scope loads,
    // all issued before any is summed, and sums them in split order.
    const size_t ct = static_cast<size_t>(item) * a.tiles + tile;
    const size_t tf = static_cast<size_t>(kMaxGemvRows) * TW;
    float* base = a.partials + ct * a.S * tf;
#pragma unroll
    for (int i = 0; i < kEl; ++i) {
      const int e = static_cast<int>(threadIdx.x) + kGemvThreads * i;
      if (e / TW < nrows)
        __hip_atomic_store(base + split * tf + e, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = __hip_atomic_fetch_add(&a.counters[ct], 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      last = (prev == a.S - 1);
    }
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int i = 0; i < kEl; ++i) {
      const int e = static_cast<int>(threadIdx.x) + kGemvThreads * i;
      if (e / TW >= nrows) continue;
      float part[kMaxSplits];
#pragma unroll
      for (int s2 = 0; s2 < kMaxSplits; ++s2)
        part[s2] = s2 < a.S ? __hip_atomic_load(base + s2 * tf + e, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)
                            : 0.0f;
      float t = 0.0f;
#pragma unroll
      for (int s2 = 0; s2 < kMaxSplits; ++s2)
        if (s2 < a.S) t += part[s2];
      v[i] = t;
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.counters[ct], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();  // all reads of the per-wave buffers are done
#pragma unroll
  for (int i = 0; i < kEl; ++i) tilev[threadIdx.x + kGemvThreads * i] = v[i];
  __syncthreads();

  // Epilogue: wave w takes sub-columns j = w, w + 4, ...
  for (int j = wv; j < SUB; j += kGemvThreads / kWave) {
    if (a.mode == 0) {
      for (int r = 0; r < nrows; ++r)
        a.out[static_cast<size_t>(pos0 + r) * a.N + col0 + 64 * j] = tilev[r * TW + 64 * j + lane];
      continue;
    }
    // SwiGLU: lanes 0..31 hold gate and 32..63 up of h columns (tile*SUB + j)*32 + c.
    // Those 32 columns are one scale group of the down projection's input, so
    // its digits are formed here directly.
    const int c = lane & 31;
    const int hg = tile * SUB + j;  // h group index
    for (int r = 0; r < nrows; ++r) {
      const float gv = tilev[r * TW + 64 * j + c];
      const float uv = tilev[r * TW + 64 * j + 32 + c];
      const float h = silu(gv) * uv;
      float amax = fabsf(h);
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      const int sh = digit_shift<D>(amax);
      const uint32_t xb = biased_fixed<D>(h, ldexpf(1.0f, sh));
      const size_t prow = static_cast<size_t>(pos0 + r);
      int32_t* blk = a.hq + (static_cast<size_t>(hg) * a.R + prow) * (4 * D);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        // gather the nibbles of lanes 8j'..8j'+7 into dword (d, j')
        uint32_t nib = digit_nibble<D>(xb, d) << (4 * (c & 7));
        nib |= __shfl_xor(nib, 1);
        nib |= __shfl_xor(nib, 2);
        nib |= __shfl_xor(nib, 4);
        if (lane < 32 && (c & 7) == 0) blk[d * 4 + (c >> 3)] = static_cast<int32_t>(nib);
      }
      if (lane == 0) a.hf[static_cast<size_t>(hg) * a.R + prow] = amax > 0.0f ? ldexpf(1.0f, -sh) : 0.0f;
      if (a.h_raw != nullptr && lane < 32) {
        const size_t hi = prow * a.N + static_cast<size_t>(hg) * 32 + c;
        if (a.h_bf16)
          static_cast<uint16_t*>(a.h_raw)[hi] = f32_to_bf16(h);
        else
          static_cast<float*>(a.h_raw)[hi] = h;
      }
    }
  }
}

}  // namespace

GemvShape gemv_shape(size_t items, int N, int mode, int G, size_t max_split_tasks) {
  const int per_sub = mode == 1 ? 32 : 64;
  const double cap = W4_GEMV_TARGET_WGS;
  GemvShape best;
  double best_fill = -1.0;
  for (int sub = W4_GEMV_SUB; sub >= 1; sub >>= 1) {
    if (N % (per_sub * sub) != 0) continue;
    GemvShape sh;
    sh.sub = sub;
    sh.tiles = N / (per_sub * sub);
    const size_t tasks = items * static_cast<size_t>(sh.tiles);
    int max_s = G / (W4_GEMV_MIN_GROUPS_PER_WAVE * (kGemvThreads / kWave));
    if (max_s > kMaxSplits) max_s = kMaxSplits;
    if (tasks > max_split_tasks) max_s = 1;
    int S = static_cast<int>(cap / static_cast<double>(tasks));
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    sh.S = S;
    const double wgs = static_cast<double>(tasks) * S;
    const double rounds = wgs <= cap ? 1.0 : static_cast<double>(static_cast<size_t>((wgs + cap - 1) / cap));
    // many rounds (grouped calls size the grid for the worst case) balance by themselves
    const double fill = rounds >= 4.0 ? 1.0 : wgs / (rounds * cap);
    if (fill > best_fill * 1.05) {  // a smaller sub must fill clearly better
      best = sh;
      best_fill = fill;
    }
  }
  return best;
}

w4a16_status_t launch_gemv(const GemvArgs& a, int D, int SUB, int input, size_t num_tasks,
                           hipStream_t stream) {
  if (num_tasks == 0) return W4A16_OK;
  if (num_tasks > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  const unsigned grid = static_cast<unsigned>(num_tasks);
#define W4_GO(d, sub, in) gemv_kernel<d, sub, in><<<grid, kGemvThreads, 0, stream>>>(a)
#define W4_SUBS(d, in)                 \
  if (SUB == 4) W4_GO(d, 4, in);       \
  else if (SUB == 2) W4_GO(d, 2, in);  \
  else W4_GO(d, 1, in);
  if (D == 5) {
    if (input == kInF32) { W4_SUBS(5, kInF32) }
    else if (input == kInBF16) { W4_SUBS(5, kInBF16) }
    else { W4_SUBS(5, kInDigits) }
  } else {
    if (input == kInF32) { W4_SUBS(4, kInF32) }
    else if (input == kInBF16) { W4_SUBS(4, kInBF16) }
    else { W4_SUBS(4, kInDigits) }
  }
#undef W4_SUBS
#undef W4_GO
  return launch_status();
}

}  // namespace w4
