// MFMA tile GEMM with exact INT4 codes for row counts above the GEMV range.
//
// y[m][n] = sum_g s[g][n] * sum_{k in g} x[m][k] * q[k][n]   (page "The Weight
// of Precision: Building Native INT4 Quantization for a Custom Speculative
// Decoding Engine", section "The Kernel: w4a16_gemm").
//
// One v_mfma_f32_16x16x32_f16 spans exactly one 32-row scale group: B holds
// the exact codes (codes_f16), A the f16 pieces of the rescaled activations
// (mfma.h), and the group's 16x16 result is scaled by s[g][n] on the float32
// accumulators.  A tile is 64 rows x 256 weight columns; the activation
// pieces of a window of groups are staged once in LDS and shared by the four
// waves, each of which streams its own 64 columns of codes: one 16-byte
// GROUPED slot per lane and group (a contiguous kilobyte per wave load), whose
// four words are column lc of the four MFMA blocks.
#include "mfma.h"
#include "mfma_ops.h"

namespace w4 {
namespace {

constexpr int kGw = 4;       // groups per staged activation window
constexpr int kRowPad = 40;  // halves per staged row of 32 (80-byte stride)

// ------------------------------------------------------------ activation pieces

// One workgroup per row.  Pass 1: the row's largest magnitude; pass 2: pieces
// of x * 2^e, each block of 8 in the order 0,4,1,5,2,6,3,7.
template <typename XT, int P>
__global__ __launch_bounds__(256) void mfma_prep_kernel(const XT* __restrict__ x, int R, int Mp,
                                                        int K, const int* __restrict__ gather,
                                                        int top_k, const int* __restrict__ need,
                                                        _Float16* __restrict__ ap,
                                                        float* __restrict__ rs) {
  __shared__ float red[256];
  const int row = blockIdx.x;
  if (need != nullptr && (row >= R || need[row] == 0)) return;
  long src = row < R ? row : -1;
  if (src >= 0 && gather != nullptr) {
    const int pr = gather[row];
    src = pr < 0 ? -1 : pr / top_k;
  }
  const XT* xr = x + (src < 0 ? 0 : src) * static_cast<size_t>(K);
  float amax = 0.0f;
  if (src >= 0)
    for (int k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(load_act(xr, k)));
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (static_cast<int>(threadIdx.x) < o) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + o]);
    __syncthreads();
  }
  amax = red[0];
  int e = 0;
  if (amax > 0.0f) {
    e = 14 - ilogbf(amax);
    e = e > 100 ? 100 : (e < -100 ? -100 : e);
  }
  const float scale = (src >= 0 && amax > 0.0f) ? ldexpf(1.0f, e) : 0.0f;
  if (threadIdx.x == 0) rs[row] = scale > 0.0f ? ldexpf(1.0f, -e) : 0.0f;
  for (int b = threadIdx.x; b < K / 8; b += 256) {
    half8 h0, h1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = scale == 0.0f ? 0.0f : load_act(xr, 8 * b + kCodeOrder[i]) * scale;
      const _Float16 hi = static_cast<_Float16>(v);
      h0[i] = hi;
      if (P == 2) h1[i] = static_cast<_Float16>(v - static_cast<float>(hi));
    }
    *reinterpret_cast<half8*>(ap + static_cast<size_t>(row) * K + 8 * b) = h0;
    if (P == 2) *reinterpret_cast<half8*>(ap + (static_cast<size_t>(Mp) + row) * K + 8 * b) = h1;
  }
}

// ------------------------------------------------------------ the MFMA kernel

template <int P>
struct MfmaLds {
  _Float16 a[P][kGw][kMfmaRows][kRowPad];
};

template <int P>
__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(const MfmaArgs a) {
  __shared__ MfmaLds<P> lds;
  __shared__ int last;
  const int task = blockIdx.x;
  const int split = task % a.S;
  const int rest = task / a.S;
  const int tile = rest % a.tiles;
  const int item = rest / a.tiles;
  int expert = 0, pos0, nrows;
  if (a.dense_rows > 0) {
    pos0 = item * kMfmaRows;
    nrows = min(kMfmaRows, a.dense_rows - pos0);
  } else {
    if (item >= *a.n_items) return;
    const int4 it = a.items[item];
    expert = it.x;
    pos0 = it.y;
    nrows = it.z;
  }
  const int wv = wave_id();
  const int lane = lane_id();
  const int lc = lane & 15, kb = lane >> 4;
  const uint32_t magic = magic_vgpr();

  // The lane reads one 16-byte GROUPED slot per group: word kb of four
  // adjacent columns col0 .. col0 + 3, which are column lc of MFMA blocks
  // cb = 0..3.  Plain: the wave's 64-column block, slot 16kb + lc.  SwiGLU:
  // the wave's 32 h columns h0 .. h0 + 31, lanes lc < 8 from gate and lanes
  // lc >= 8 from up (the same h columns), so a lane pair (lc, lc + 8) holds
  // gate and up of one output.
  int mat, col0, chunk;
  bool wave_ok;
  if (a.mode == 1) {
    const int h0 = tile * 128 + wv * 32;
    wave_ok = h0 < a.N;
    mat = lc >> 3;
    col0 = h0 + 4 * (lc & 7);
    chunk = (h0 >> 6) * 64 + 16 * kb + ((h0 >> 5) & 1) * 8 + (lc & 7);
  } else {
    const int c0 = tile * kMfmaCols + wv * 64;
    wave_ok = c0 < a.N;
    mat = 0;
    col0 = c0 + 4 * lc;
    chunk = c0 + 16 * kb + lc;
  }
  const size_t ebase = static_cast<size_t>(expert) * a.expert_stride;
  const u32x4* wp = (mat ? a.qw1 : a.qw0) + ebase + (wave_ok ? chunk : 0);
  const float* sp = (mat ? a.sc1 : a.sc0) + ebase + (wave_ok ? col0 : 0);
  const size_t gstride = static_cast<size_t>(a.N);  // chunks (and scales) per group row

  f32x4 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int g_lo = split * a.gps;
  const int g_hi = min(a.G, g_lo + a.gps);
  for (int gw = g_lo; gw < g_hi; gw += kGw) {
    const int nw = min(kGw, g_hi - gw);
    // stage the pieces of rows pos0..pos0+63, groups gw..gw+nw-1: 16-byte units
    const int units = P * nw * kMfmaRows * 4;
    for (int u = threadIdx.x; u < units; u += kMfmaThreads) {
      const int q4 = u & 3;
      const int r = (u >> 2) % kMfmaRows;
      const int gl = (u >> 2) / kMfmaRows % nw;
      const int p = (u >> 2) / kMfmaRows / nw;
      const half8 v = *reinterpret_cast<const half8*>(
          a.ap + (static_cast<size_t>(p) * a.Mp + pos0 + r) * a.K + static_cast<size_t>(gw + gl) * kGroup + 8 * q4);
      *reinterpret_cast<half8*>(&lds.a[p][gl][r][8 * q4]) = v;
    }
    __syncthreads();
    if (wave_ok) {
      u32x4 wn = __builtin_nontemporal_load(wp + static_cast<size_t>(gw) * gstride);
      f32x4 sn = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp + static_cast<size_t>(gw) * gstride));
      for (int gl = 0; gl < nw; ++gl) {
        const u32x4 wc = wn;
        const f32x4 sc = sn;
        if (gl + 1 < nw) {
          wn = __builtin_nontemporal_load(wp + static_cast<size_t>(gw + gl + 1) * gstride);
          sn = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4*>(sp + static_cast<size_t>(gw + gl + 1) * gstride));
        }
        half8 bq[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) bq[cb] = codes_f16(wc[cb], magic);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          half8 af[P];
#pragma unroll
          for (int p = 0; p < P; ++p)
            af[p] = *reinterpret_cast<const half8*>(&lds.a[p][gl][rb * 16 + lc][8 * kb]);
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[0], bq[cb], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            if (P == 2) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[1], bq[cb], d, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rb][cb][i] = fmaf(sc[cb], d[i], acc[rb][cb][i]);
          }
        }
      }
    }
    __syncthreads();
  }

  // split-K: write-through partials, agent-scope arrival counter, the last
  // workgroup sums the partials in split order (see the GEMV kernel)
  if (a.S > 1) {
    const size_t ct = static_cast<size_t>(item) * a.tiles + tile;
    const size_t tf = static_cast<size_t>(kMfmaRows) * kMfmaCols;
    float* base = a.partials + ct * a.S * tf;
    if (wave_ok) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rb * 16 + 4 * kb + i;
            __hip_atomic_store(base + split * tf + r * kMfmaCols + wv * 64 + cb * 16 + lc, acc[rb][cb][i],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      last = (__hip_atomic_fetch_add(&a.counters[ct], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              a.S - 1);
    __syncthreads();
    if (!last) return;
    if (wave_ok) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = rb * 16 + 4 * kb + i;
            const float* pp = base + r * kMfmaCols + wv * 64 + cb * 16 + lc;
            float t = 0.0f;
            for (int s2 = 0; s2 < a.S; ++s2)
              t += __hip_atomic_load(pp + s2 * tf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            acc[rb][cb][i] = t;
          }
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.counters[ct], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!wave_ok) return;

#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + 4 * kb + i;
      const bool live = r < nrows;
      const size_t prow = static_cast<size_t>(pos0 + (live ? r : 0));
      const float f = live ? a.rs[prow] : 0.0f;
      if (a.mode == 0) {
        if (live) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) a.out[prow * a.N + col0 + cb] = acc[rb][cb][i] * f;
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const float up = __shfl_xor(acc[rb][cb][i], 8);  // every lane takes part
          if (live && lc < 8) {
            const float h = silu(acc[rb][cb][i] * f) * (up * f);
            const size_t hi = prow * a.N + col0 + cb;
            if (a.h_bf16)
              static_cast<uint16_t*>(a.h)[hi] = f32_to_bf16(h);
            else
              static_cast<float*>(a.h)[hi] = h;
          }
        }
      }
    }
}

}  // namespace

w4a16_status_t launch_mfma_prep(const void* x, w4a16_dtype_t xt, int R, int Mp, int K, int P,
                                const int* gather, int top_k, const int* need, _Float16* ap,
                                float* rs, hipStream_t stream) {
  if (Mp == 0) return W4A16_OK;
  if (xt == W4A16_F32 && P == 2)
    mfma_prep_kernel<float, 2><<<Mp, 256, 0, stream>>>(static_cast<const float*>(x), R, Mp, K, gather,
                                                       top_k, need, ap, rs);
  else if (xt == W4A16_F32)
    mfma_prep_kernel<float, 1><<<Mp, 256, 0, stream>>>(static_cast<const float*>(x), R, Mp, K, gather,
                                                       top_k, need, ap, rs);
  else if (P == 2)
    mfma_prep_kernel<uint16_t, 2><<<Mp, 256, 0, stream>>>(static_cast<const uint16_t*>(x), R, Mp, K,
                                                          gather, top_k, need, ap, rs);
  else
    mfma_prep_kernel<uint16_t, 1><<<Mp, 256, 0, stream>>>(static_cast<const uint16_t*>(x), R, Mp, K,
                                                          gather, top_k, need, ap, rs);
  return launch_status();
}

w4a16_status_t launch_mfma(const MfmaArgs& a, int P, size_t num_tasks, hipStream_t stream) {
  if (num_tasks == 0) return W4A16_OK;
  if (num_tasks > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  const unsigned grid = static_cast<unsigned>(num_tasks);
  if (P == 2)
    mfma_kernel<2><<<grid, kMfmaThreads, 0, stream>>>(a);
  else
    mfma_kernel<1><<<grid, kMfmaThreads, 0, stream>>>(a);
  return launch_status();
}

}  // namespace w4
