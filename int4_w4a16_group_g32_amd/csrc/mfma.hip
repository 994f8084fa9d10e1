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
#include <type_traits>

#include "mfma.h"
#include "gemv.h"  // kMaxSplits

#include <hip/hip_ext.h>
#include "mfma_ops.h"

namespace w4 {
namespace {

constexpr int kGw = 4;           // groups per staged activation window (double-buffered)
constexpr int kTileRing = 2 * kGw;  // groups of codes in flight per wave (two windows)
// Grouped launches (MoE items) hold many workgroups: they run three waves per
// SIMD with a ring of one window, which the register budget of three waves
// allows; dense launches keep two waves and two windows.
constexpr int kGroupedRing = kGw;
constexpr int kPrepThreads = 1024;
#ifndef W4_PREP_WAVE
#define W4_PREP_WAVE 1
#endif
constexpr bool kPrepWave = W4_PREP_WAVE != 0;  // one wave per row for rows of at most 4096 values

// ------------------------------------------------------------ activation pieces

template <typename XT>
__device__ __forceinline__ void load8(const XT* xr, int b, float v[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* xr, int b, float v[8]) {
  const float4 u0 = reinterpret_cast<const float4*>(xr)[2 * b];
  const float4 u1 = reinterpret_cast<const float4*>(xr)[2 * b + 1];
  v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
  v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
}
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* xr, int b, float v[8]) {
  const uint4 u = reinterpret_cast<const uint4*>(xr)[b];
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __uint_as_float(w[j] << 16);
    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

// One workgroup per row.  Pass 1: the row's largest magnitude; pass 2: pieces
// of x * 2^e, each block of 8 in the order 0,4,1,5,2,6,3,7.  A thread takes
// blocks of 8 consecutive activations (one or two 16-byte loads).
template <typename XT, int P>
__global__ __launch_bounds__(kPrepThreads) void mfma_prep_kernel(const XT* __restrict__ x, int R, int Mp,
                                                                 int K, const int* __restrict__ gather,
                                                                 int top_k, const int* __restrict__ need,
                                                                 _Float16* __restrict__ ap,
                                                                 float* __restrict__ rs) {
  __shared__ float red[kPrepThreads / kWave];
  const int row = blockIdx.x;
  if (need != nullptr && (row >= R || need[row] == 0)) return;
  long src = row < R ? row : -1;
  if (src >= 0 && gather != nullptr) {
    const int pr = gather[row];
    src = pr < 0 ? -1 : pr / top_k;
  }
  const XT* xr = x + (src < 0 ? 0 : src) * static_cast<size_t>(K);
  const int nb = K / 8;
  float amax = 0.0f;
  if (src >= 0) {
    for (int b = threadIdx.x; b < nb; b += kPrepThreads) {
      float v[8];
      load8<XT>(xr, b, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (lane_id() == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = 0.0f;
#pragma unroll
  for (int w = 0; w < kPrepThreads / kWave; ++w) amax = fmaxf(amax, red[w]);
  int e = 0;
  if (amax > 0.0f) {
    int lg = ilogbf(amax);
    lg = lg > 120 ? 120 : (lg < -120 ? -120 : lg);
    e = 14 - lg;
  }
  const float scale = (src >= 0 && amax > 0.0f) ? ldexpf(1.0f, e) : 0.0f;
  if (threadIdx.x == 0) rs[row] = scale > 0.0f ? ldexpf(1.0f, -e) : 0.0f;
  for (int b = threadIdx.x; b < nb; b += kPrepThreads) {
    float v[8];
    if (scale != 0.0f) {
      load8<XT>(xr, b, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    half8 h0, h1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = v[kCodeOrder[i]] * scale;
      const _Float16 hi = static_cast<_Float16>(t);
      h0[i] = hi;
      if (P == 2) h1[i] = static_cast<_Float16>(t - static_cast<float>(hi));
    }
    *reinterpret_cast<half8*>(ap + static_cast<size_t>(row) * K + 8 * b) = h0;
    if (P == 2) *reinterpret_cast<half8*>(ap + (static_cast<size_t>(Mp) + row) * K + 8 * b) = h1;
  }
}

// The same pieces for rows of at most 64 * kB blocks of 8: one wave per row,
// four rows per workgroup.  Each lane keeps its kB blocks in registers
// between the two passes, and the largest magnitude needs only a wave
// reduction, so short rows (the down projection's h of an expert, K = 2048)
// no longer leave most of a 1024-thread workgroup idle.
constexpr int kPrepWaveThreads = 256;

template <typename XT, int P, int kB>
__global__ __launch_bounds__(kPrepWaveThreads) void mfma_prep_wave_kernel(const XT* __restrict__ x, int R, int Mp,
                                                                          int K, const int* __restrict__ gather,
                                                                          int top_k, const int* __restrict__ need,
                                                                          _Float16* __restrict__ ap,
                                                                          float* __restrict__ rs) {
  const int row = static_cast<int>(blockIdx.x) * (kPrepWaveThreads / kWave) + wave_id();
  if (row >= Mp) return;
  if (need != nullptr && (row >= R || need[row] == 0)) return;
  long src = row < R ? row : -1;
  if (src >= 0 && gather != nullptr) {
    const int pr = gather[row];
    src = pr < 0 ? -1 : pr / top_k;
  }
  const XT* xr = x + (src < 0 ? 0 : src) * static_cast<size_t>(K);
  const int nb = K / 8;
  const int lane = lane_id();
  float v[kB][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    const int b = lane + kWave * i;
    if (src >= 0 && b < nb) {
      load8<XT>(xr, b, v[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  int e = 0;
  if (amax > 0.0f) {
    int lg = ilogbf(amax);
    lg = lg > 120 ? 120 : (lg < -120 ? -120 : lg);
    e = 14 - lg;
  }
  const float scale = (src >= 0 && amax > 0.0f) ? ldexpf(1.0f, e) : 0.0f;
  if (lane == 0) rs[row] = scale > 0.0f ? ldexpf(1.0f, -e) : 0.0f;
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    const int b = lane + kWave * i;
    if (b >= nb) break;
    half8 h0, h1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // a row without a nonzero value stores +0 pieces, as the workgroup form does
      const float t = scale != 0.0f ? v[i][kCodeOrder[j]] * scale : 0.0f;
      const _Float16 hi = static_cast<_Float16>(t);
      h0[j] = hi;
      if (P == 2) h1[j] = static_cast<_Float16>(t - static_cast<float>(hi));
    }
    *reinterpret_cast<half8*>(ap + static_cast<size_t>(row) * K + 8 * b) = h0;
    if (P == 2) *reinterpret_cast<half8*>(ap + (static_cast<size_t>(Mp) + row) * K + 8 * b) = h1;
  }
}

template <int kB>
void launch_prep_wave(const void* x, w4a16_dtype_t xt, int R, int Mp, int K, int P, const int* gather, int top_k,
                      const int* need, _Float16* ap, float* rs, hipStream_t stream, hipEvent_t start,
                      hipEvent_t stop) {
  const float* xf = static_cast<const float*>(x);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const dim3 g((Mp + kPrepWaveThreads / kWave - 1) / (kPrepWaveThreads / kWave)), b(kPrepWaveThreads);
  if (xt == W4A16_F32 && P == 2)
    hipExtLaunchKernelGGL(mfma_prep_wave_kernel<float, 2, kB>, g, b, 0, stream, start, stop, 0, xf, R, Mp, K,
                          gather, top_k, need, ap, rs);
  else if (xt == W4A16_F32)
    hipExtLaunchKernelGGL(mfma_prep_wave_kernel<float, 1, kB>, g, b, 0, stream, start, stop, 0, xf, R, Mp, K,
                          gather, top_k, need, ap, rs);
  else if (P == 2)
    hipExtLaunchKernelGGL(mfma_prep_wave_kernel<uint16_t, 2, kB>, g, b, 0, stream, start, stop, 0, xb, R, Mp, K,
                          gather, top_k, need, ap, rs);
  else
    hipExtLaunchKernelGGL(mfma_prep_wave_kernel<uint16_t, 1, kB>, g, b, 0, stream, start, stop, 0, xb, R, Mp, K,
                          gather, top_k, need, ap, rs);
}

// ------------------------------------------------------------ the MFMA kernel

// Activation window: 16-byte unit (p, gl, row, kb) at a_off(); k blocks are
// XOR-swizzled by row so the 16 rows one ds_read_b128 touches fall in
// distinct banks.
template <int P>
constexpr int kWinUnits = P * kGw * kMfmaRows * 4;

__device__ __forceinline__ int a_off(int p, int gl, int row, int kb) {
  return ((p * kGw + gl) * kMfmaRows + row) * 4 + (kb ^ ((row >> 2) & 3));
}

template <int P>
struct MfmaLds {
  uint4 a[2][kWinUnits<P>];  // double buffer
};

// Thread t loads units t, t + 256, ...: unit u holds k block u & 3 of tile
// row 4 * (u >> 6) + ((u >> 2) & 3) (in piece plane u >> 10) and window group
// (u >> 4) & 3, so 16 consecutive threads take four rows' 64 bytes of one
// group, and their stores (four rows times four k blocks) fall in 16 distinct
// bank groups.  A thread keeps one window group and one k block throughout.
// The loads are unconditional (clamped addresses); groups past the split's
// end are zeroed when the window is stored, so the tail needs no masking.  A
// load under a branch, or a use of its value before the window's groups are
// done, would make the compiler's wait cover the code ring as well.
// The thread's units cover four tile rows, the same in every window and
// piece plane: srow[j] is the piece row of tile row row_of_unit(j).
constexpr int kUnitRows = 4;
struct WinUnit {
  int kb, gl, row, p;
};
__device__ __forceinline__ WinUnit win_unit(int i) {
  const int u = static_cast<int>(threadIdx.x) + kMfmaThreads * i;
  return WinUnit{u & 3, (u >> 4) & 3, (4 * (u >> 6) + ((u >> 2) & 3)) % kMfmaRows, u >> 10};
}
__device__ __forceinline__ int row_of_unit(int i) { return win_unit(i).row; }

template <int P>
__device__ __forceinline__ void load_a_window(const MfmaArgs& a, const int srow[kUnitRows], int gw, int g_hi,
                                              uint4 r[kWinUnits<P> / kMfmaThreads]) {
  static_assert(kGw == 4 && kMfmaThreads == 256 && kMfmaRows == 64, "the unit mapping assumes these sizes");
#pragma unroll
  for (int i = 0; i < kWinUnits<P> / kMfmaThreads; ++i) {
    const WinUnit w = win_unit(i);
    r[i] = *reinterpret_cast<const uint4*>(a.ap + (static_cast<size_t>(w.p) * a.Mp + srow[i % kUnitRows]) * a.K +
                                           static_cast<size_t>(min(gw + w.gl, g_hi - 1)) * kGroup + 8 * w.kb);
  }
}

template <int P>
__device__ __forceinline__ void store_a_window(uint4* buf, int gw, int g_hi,
                                               const uint4 r[kWinUnits<P> / kMfmaThreads]) {
#pragma unroll
  for (int i = 0; i < kWinUnits<P> / kMfmaThreads; ++i) {
    const WinUnit w = win_unit(i);
    buf[a_off(w.p, w.gl, w.row, w.kb)] = gw + w.gl < g_hi ? r[i] : make_uint4(0, 0, 0, 0);
  }
}

struct TileCodes {
  u32x4 w;  // word kb of the lane's four columns
  f32x4 s;  // their scales
};

// Raw buffer resources: a wave-uniform base and size in scalar registers, so
// a load takes one 32-bit lane offset and a scalar offset for the group (no
// 64-bit address arithmetic per load).  The hardware's size check covers the
// lane offset only, so the scalar offsets stay inside the buffer by
// construction (groups are clamped to the split's last one).
constexpr int kBufFlags = 0x00020000;  // dword 3 of a raw buffer resource on gfx9
constexpr int kNt = 2;                 // nontemporal: the codes and scales are read once

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufFlags);
}

// The codes and scales of split-relative group gr (clamped to the split's last
// group gr_last): the code buffer starts at the split's first group, the scale
// buffer at its first scale row s_lo.
struct CodeSrc {
  __amdgpu_buffer_rsrc_t w, s;
  int wvoff, svoff;  // lane offsets (bytes)
  int wstep, sstep;  // bytes per group row of codes, per scale row
  int g_lo, s_lo, gshift;
};

__device__ __forceinline__ void load_tile_codes(const CodeSrc& c, int gr, int gr_last, TileCodes& t) {
  const int g = min(gr, gr_last);
  t.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.w, c.wvoff, g * c.wstep, kNt));
  t.s = __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(c.s, c.svoff, (((c.g_lo + g) >> c.gshift) - c.s_lo) * c.sstep, kNt));
}

// One group of the tile: the live row blocks (nrb of 4, wave-uniform) x 4
// column blocks.
//
// Two pieces (float32 activations): B holds the exact codes and each group's
// 16x16 result is scaled by s[g][n] on the float32 accumulators, so the scale
// is applied exactly once, in float32.
//
// One piece (bf16 activations): the scale is folded into B, which holds
// f16(q * f16(s * 2^c)) for a per-lane, per-column-block power of two 2^c
// (the lanes that share a column see the same scales and so keep the same
// c), and the MFMA accumulates straight into the accumulators; the epilogue
// multiplies by 2^-c.  c starts so that the largest scale of the split's first
// ring of groups lands in [1/2, 1) (2^138 if they are all zero); a later
// group whose scaled value would reach 2^12 (where q * s could leave the f16
// range) moves c to bring it to [1/2, 1) and rescales that column block's
// accumulators by the same power of two, so no product overflows.  Each
// weight is then rounded twice in f16 (about 2^-11 relative each); a group
// whose scale lies more than 2^14 below the anchor keeps an absolute precision
// of about 2^-25 of the anchor instead, and float32 scales below the normal
// range (2^-126) are carried with reduced precision.
template <int P>
__device__ __forceinline__ void mma_tile_group(const uint4* buf, int gl, int lc, int kb, uint32_t magic,
                                               const TileCodes& c, int nrb, int cexp[4], f32x4 acc[4][4]) {
  half8 bq[4];
  if (P == 1) {
    f32x4 sp;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) sp[cb] = ldexpf(c.s[cb], cexp[cb]);
    const float m = fmaxf(fmaxf(fabsf(sp[0]), fabsf(sp[1])), fmaxf(fabsf(sp[2]), fabsf(sp[3])));
    if (__builtin_amdgcn_ballot_w64(m >= 4096.0f) != 0) {  // rare: re-anchor
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        // from the raw scale, so a scaled value that overflowed to inf still
        // gets its anchor
        const bool move = fabsf(sp[cb]) >= 4096.0f;
        const int cn = move ? -__builtin_amdgcn_frexp_expf(c.s[cb]) : cexp[cb];
        const int d = cexp[cb] - cn;
        cexp[cb] = cn;
        sp[cb] = ldexpf(c.s[cb], cn);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][cb][i] = ldexpf(acc[rb][cb][i], -d);
      }
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const _Float16 h = static_cast<_Float16>(sp[cb]);
      bq[cb] = codes_f16(c.w[cb], magic) * half8{h, h, h, h, h, h, h, h};
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) bq[cb] = codes_f16(c.w[cb], magic);
  }
  // all row blocks' fragments are read (the window holds 64 rows), so one
  // wait covers them; only the MFMAs of dead row blocks are skipped
  half8 af[4][P];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int p = 0; p < P; ++p) af[rb][p] = __builtin_bit_cast(half8, buf[a_off(p, gl, rb * 16 + lc, kb)]);
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb < nrb) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        if (P == 1) {
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[rb][0], bq[cb], acc[rb][cb], 0, 0, 0);
        } else {
          f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[rb][0], bq[cb], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[rb][P - 1], bq[cb], d, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][cb][i] = fmaf(c.s[cb], d[i], acc[rb][cb][i]);
        }
      }
    }
  }
}

// The end of a tile task: the split-K sum (write-through partials, an
// agent-scope arrival counter, and the last workgroup sums the partials in
// split order), then the plain or SwiGLU output.  Every thread of the
// workgroup calls it.
template <int P, int kWaves, bool kDefer>
__device__ __forceinline__ void tile_finish(const MfmaArgs& a, MfmaLds<P>& lds, int* last, f32x4 acc[4][4],
                                            int item, int tile, int split, int pos0, int nrows, int wv, int lane,
                                            int kb, bool wave_ok, int col0) {
  if (kDefer) {
    // deferred split-K: this split's sums
    if (!wave_ok) return;
    const int mat = a.mode == 1 ? wv >> 1 : 0;
    float* base = a.planes + (static_cast<size_t>(split * (a.mode == 1 ? 2 : 1) + mat) * a.plane_rows + pos0) *
                                 a.plane_ld + col0;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + 4 * kb + i;
        if (r < nrows) {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) base[static_cast<size_t>(r) * a.plane_ld + cb] = acc[rb][cb][i];
        }
      }
    return;
  }
  // Split-K: write-through partials, an agent-scope arrival counter, and the
  // last workgroup sums the partials in split order (the GEMV kernel's
  // scheme, with the same reliance on gfx950's write-through agent-scope
  // atomics in place of release/acquire ordering).  A partial tile is stored
  // element-major, [j][thread] with j = (rb * 4 + cb) * 4 + i, so every store
  // and load instruction covers 256 contiguous bytes, and the readback keeps
  // two splits' worth (128 loads per thread) in flight at a time.
  if (a.S > 1) {
    const size_t ct = static_cast<size_t>(item) * a.tiles + tile;
    const size_t tf = static_cast<size_t>(kMfmaRows) * kMfmaCols;
    float* base = a.partials + ct * a.S * tf + threadIdx.x;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(base + split * tf + ((rb * 4 + cb) * 4 + i) * kMfmaThreads, acc[rb][cb][i],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0)
      *last = (__hip_atomic_fetch_add(&a.counters[ct], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              a.S - 1);
    __syncthreads();
    if (!*last) return;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // partials in flight per round: two (128 loads per thread) at two waves
    // per SIMD, one at three (its register budget)
    constexpr int kB = kWaves >= 3 ? 1 : 2;
    for (int s0 = 0; s0 < a.S; s0 += kB) {
      float p[kB][64];
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        const float* ps = base + static_cast<size_t>(min(s0 + b, a.S - 1)) * tf;
#pragma unroll
        for (int e = 0; e < 64; ++e)
          p[b][e] = __hip_atomic_load(ps + e * kMfmaThreads, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        if (s0 + b < a.S) {
#pragma unroll
          for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[rb][cb][i] += p[b][(rb * 4 + cb) * 4 + i];
        }
      }
    }
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.counters[ct], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (a.mode == 1) {
    // The up waves hand their sums to the gate waves of the same columns
    // through LDS (the window buffers are free now), element-major like the
    // partial tiles.
    float* xu = reinterpret_cast<float*>(&lds.a[0][0]);
    static_assert(sizeof(MfmaLds<P>) >= 2 * 64 * 64 * sizeof(float), "the up sums must fit in the windows");
    __syncthreads();  // every wave is done with the windows
    if (wv >= 2) {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) xu[(((wv & 1) * 64 + (rb * 4 + cb) * 4 + i) << 6) + lane] = acc[rb][cb][i];
    }
    __syncthreads();
    if (wv >= 2 || !wave_ok) return;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rb * 16 + 4 * kb + i;
        if (r < nrows) {
          const size_t prow = static_cast<size_t>(pos0 + r);
          const float f = a.rs[a.arow != nullptr ? a.arow[prow] / a.arow_div : prow];
          float hv[4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) {
            const float up = xu[(((wv & 1) * 64 + (rb * 4 + cb) * 4 + i) << 6) + lane];
            hv[cb] = silu(acc[rb][cb][i] * f) * (up * f);
          }
          if (a.h_bf16) {
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.h) + prow * a.N + col0) =
                make_uint2(f32_to_bf16(hv[0]) | (static_cast<uint32_t>(f32_to_bf16(hv[1])) << 16),
                           f32_to_bf16(hv[2]) | (static_cast<uint32_t>(f32_to_bf16(hv[3])) << 16));
          } else {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) a.h[prow * a.N + col0 + cb] = hv[cb];
          }
        }
      }
    return;
  }
  if (!wave_ok) return;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + 4 * kb + i;
      if (r < nrows) {
        const size_t prow = static_cast<size_t>(pos0 + r);
        const float f = a.rs[a.arow != nullptr ? a.arow[prow] / a.arow_div : prow];
        if (a.out_bf16) {
          uint32_t b[4];
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) b[cb] = f32_to_bf16(acc[rb][cb][i] * f);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + prow * a.N + col0) =
              make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
        } else {
#pragma unroll
          for (int cb = 0; cb < 4; ++cb) a.out[prow * a.N + col0 + cb] = acc[rb][cb][i] * f;
        }
      }
    }
}

template <int P, int R, int kWaves, bool kDefer = false>
__global__ __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(kWaves, kWaves)))
void mfma_kernel(const MfmaArgs a) {
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
    if (item >= __builtin_amdgcn_readfirstlane(*a.n_items)) return;
    const int4 it = a.items[item];
    // the item is the same for the whole workgroup: keep it in scalar registers
    expert = __builtin_amdgcn_readfirstlane(it.x);
    pos0 = __builtin_amdgcn_readfirstlane(it.y);
    nrows = __builtin_amdgcn_readfirstlane(it.z);
  }
  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const int lane = lane_id();
  const int lc = lane & 15, kb = lane >> 4;
  const uint32_t magic = magic_vgpr();

  // The lane reads one 16-byte GROUPED slot per group: word kb of four
  // adjacent columns col0 .. col0 + 3, which are column lc of MFMA blocks
  // cb = 0..3, so a wave load is one contiguous kilobyte of its 64-column
  // block.  Plain: wave wv streams columns c0 = 256 tile + 64 wv.  SwiGLU: the
  // tile is 128 h columns; waves 0 and 1 stream gate columns c0 = 128 tile +
  // 64 (wv & 1), waves 2 and 3 the same columns of up, and the epilogue pairs
  // them through LDS.
  const int mat = a.mode == 1 ? wv >> 1 : 0;
  const int c0 = a.mode == 1 ? tile * (kMfmaCols / 2) + (wv & 1) * 64 : tile * kMfmaCols + wv * 64;
  const bool wave_ok = c0 < a.N;
  const int col0 = c0 + 4 * lc;
  const size_t ebase = static_cast<size_t>(expert) * a.expert_stride;
  const bool xe = expert + 1 == a.extra_plus1;
  const u32x4* qb = xe ? (mat ? a.qw1x : a.qw0x) : (mat ? a.qw1 : a.qw0) + ebase;
  const float* sb = xe ? (mat ? a.sc1x : a.sc0x) : (mat ? a.sc1 : a.sc0) + (ebase >> a.gshift);

  f32x4 acc[4][4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int g_lo = split * a.gps;
  const int g_hi = min(a.G, g_lo + a.gps);
  const int g_last = g_hi - 1;
  const int nwin = (g_hi - g_lo + kGw - 1) / kGw;
  // Codes and scales of the split.  A wave past the matrix's last column
  // streams column block 0 and stores nothing, so every load below is
  // unconditional.
  CodeSrc cs;
  {
    const size_t row_bytes = static_cast<size_t>(a.N) * 16;  // one group row of GROUPED slots
    const int s_lo = g_lo >> a.gshift, s_hi = g_last >> a.gshift;
    cs.w = tile_rsrc(qb + static_cast<size_t>(g_lo) * a.N, static_cast<size_t>(g_hi - g_lo) * row_bytes);
    cs.s = tile_rsrc(sb + static_cast<size_t>(s_lo) * a.N, static_cast<size_t>(s_hi - s_lo + 1) * a.N * 4);
    cs.wvoff = (wave_ok ? c0 + 16 * kb + lc : 16 * kb + lc) * 16;
    cs.svoff = (wave_ok ? col0 : 4 * lc) * 4;
    cs.wstep = a.N * 16;
    cs.sstep = a.N * 4;
    cs.g_lo = g_lo;
    cs.s_lo = s_lo;
    cs.gshift = a.gshift;
  }
  const int gr_last = g_last - g_lo;
  uint4 ra[kWinUnits<P> / kMfmaThreads];
  // ring of R groups of codes in flight (one or two windows): group g_lo + i
  // sits in slot i % R, so a window always uses the same slots
  static_assert(R == kGw || R == 2 * kGw, "ring of one or two windows");
  TileCodes ring[R];
  int srow[kUnitRows];
#pragma unroll
  for (int j = 0; j < kUnitRows; ++j) {
    const int pr = pos0 + row_of_unit(j);
    srow[j] = a.arow != nullptr ? a.arow[min(pr, a.arow_n - 1)] / a.arow_div : pr;
  }
  load_a_window<P>(a, srow, g_lo, g_hi, ra);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    load_tile_codes(cs, j, gr_last, ring[j]);
    __builtin_amdgcn_sched_barrier(0);  // issue order = use order
  }
  // live 16-row blocks of the tile (items hold 1 .. 64 rows), a scalar
  const int nrb = __builtin_amdgcn_readfirstlane((nrows + 15) >> 4);
  // one piece: the per-column-block anchors (see mma_tile_group)
  int cexp[4] = {0, 0, 0, 0};
  if (P == 1) {
    f32x4 mx = ring[0].s;
#pragma unroll
    for (int j = 1; j < R; ++j)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) mx[cb] = fmaxf(fabsf(mx[cb]), fabsf(ring[j].s[cb]));
    // an all-zero start takes the first nonzero group's anchor on arrival:
    // 2^138 lifts every normal float32 scale to 2^12 or more
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) cexp[cb] = mx[cb] != 0.0f ? -__builtin_amdgcn_frexp_expf(fabsf(mx[cb])) : 138;
  }
  store_a_window<P>(lds.a[0], g_lo, g_hi, ra);
  __syncthreads();
  // Window wi uses LDS buffer and ring half h = wi % 2.  The loop body is two
  // whole windows and an odd last window runs after it, so every path into
  // the loop header has the same loads outstanding (with a conditional second
  // window the compiler's waits would drain half the ring at every header).
  auto window = [&](int wi, auto hc) {
    constexpr int h = decltype(hc)::value;
    const int gw = g_lo + wi * kGw;
    load_a_window<P>(a, srow, gw + kGw, g_hi, ra);  // the next window, in flight
#pragma unroll
    for (int j = 0; j < kGw; ++j) {
      mma_tile_group<P>(lds.a[h], j, lc, kb, magic, ring[(kGw * h + j) % R], nrb, cexp, acc);
      load_tile_codes(cs, gw - g_lo + j + R, gr_last, ring[(kGw * h + j) % R]);
      __builtin_amdgcn_sched_barrier(0);
    }
    store_a_window<P>(lds.a[1 - h], gw + kGw, g_hi, ra);
    __syncthreads();
  };
  int w = 0;
  for (; w + 1 < nwin; w += 2) {
    window(w, std::integral_constant<int, 0>{});
    window(w + 1, std::integral_constant<int, 1>{});
  }
  if (w < nwin) window(w, std::integral_constant<int, 0>{});

  if (P == 1) {  // back to the scales' own units
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rb][cb][i] = ldexpf(acc[rb][cb][i], -cexp[cb]);
  }

  tile_finish<P, kWaves, kDefer>(a, lds, &last, acc, item, tile, split, pos0, nrows, wv, lane, kb, wave_ok, col0);
}

// ------------------------------------------------------- deferred split-K

// out[m][n..n+3] = (sum of the split planes, split order) * rs[m], or with
// rs_stride > 0 the split-order sum of planes[s] * rs[s * rs_stride + m]
// (activations scaled per row and split): one thread per four columns, every
// split's loads in flight before the sum.
__global__ __launch_bounds__(256) void plane_sum_kernel(const float* __restrict__ planes, int S, int plane_rows,
                                                        int plane_ld, const float* __restrict__ rs, int rs_stride,
                                                        int M, int N, float* __restrict__ out) {
  const int n4 = N / 4;
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<size_t>(M) * n4) return;
  const int m = static_cast<int>(idx / n4), n = static_cast<int>(idx % n4) * 4;
  const size_t sstride = static_cast<size_t>(plane_rows) * plane_ld;
  const float* p = planes + static_cast<size_t>(m) * plane_ld + n;
  f32x4 v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < S) v[s] = *reinterpret_cast<const f32x4*>(p + s * sstride);
  f32x4 t = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (rs_stride > 0) {
    float f[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      if (s < S) f[s] = rs[static_cast<size_t>(s) * rs_stride + m];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
      if (s < S) t += v[s] * f[s];
    *reinterpret_cast<f32x4*>(out + static_cast<size_t>(m) * N + n) = t;
    return;
  }
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < S) t += v[s];
  const float f = rs[m];
  *reinterpret_cast<f32x4*>(out + static_cast<size_t>(m) * N + n) = t * f;
}

// The pieces of h from the gate/up split planes, one workgroup per row:
// pass 1 sums the splits in order, forms h = silu(g * f) * (u * f), stores
// it to h and takes the row's largest magnitude; pass 2 reads the row back
// and writes its pieces (as mfma_prep_kernel).
template <int P>
__global__ __launch_bounds__(kPrepThreads) void prep_planes_kernel(const float* __restrict__ planes, int S,
                                                                   int plane_rows, int plane_ld,
                                                                   const float* __restrict__ rsx, int M, int Mp,
                                                                   int I, float* __restrict__ h,
                                                                   _Float16* __restrict__ ap,
                                                                   float* __restrict__ rs) {
  __shared__ float red[kPrepThreads / kWave];
  const int row = blockIdx.x;
  const int nb = I / 8;
  float amax = 0.0f;
  const size_t sstride = static_cast<size_t>(2) * plane_rows * plane_ld;  // one split: gate plane + up plane
  float* hr = h + static_cast<size_t>(row < M ? row : 0) * I;
  if (row < M) {
    const float f = rsx[row];
    const float* gp = planes + static_cast<size_t>(row) * plane_ld;
    const float* up = gp + static_cast<size_t>(plane_rows) * plane_ld;
    for (int b = threadIdx.x; b < nb; b += kPrepThreads) {
      f32x4 g0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, g1 = g0, u0 = g0, u1 = g0;
      for (int s = 0; s < S; ++s) {
        const size_t o = s * sstride + 8 * static_cast<size_t>(b);
        g0 += *reinterpret_cast<const f32x4*>(gp + o);
        g1 += *reinterpret_cast<const f32x4*>(gp + o + 4);
        u0 += *reinterpret_cast<const f32x4*>(up + o);
        u1 += *reinterpret_cast<const f32x4*>(up + o + 4);
      }
      f32x4 h0, h1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h0[i] = silu(g0[i] * f) * (u0[i] * f);
        h1[i] = silu(g1[i] * f) * (u1[i] * f);
        amax = fmaxf(amax, fmaxf(fabsf(h0[i]), fabsf(h1[i])));
      }
      *reinterpret_cast<f32x4*>(hr + 8 * b) = h0;
      *reinterpret_cast<f32x4*>(hr + 8 * b + 4) = h1;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (lane_id() == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();  // (also orders this workgroup's h stores before pass 2 reads them)
  amax = 0.0f;
#pragma unroll
  for (int w = 0; w < kPrepThreads / kWave; ++w) amax = fmaxf(amax, red[w]);
  int e = 0;
  if (amax > 0.0f) {
    int lg = ilogbf(amax);
    lg = lg > 120 ? 120 : (lg < -120 ? -120 : lg);
    e = 14 - lg;
  }
  const float scale = (row < M && amax > 0.0f) ? ldexpf(1.0f, e) : 0.0f;
  if (threadIdx.x == 0) rs[row] = scale > 0.0f ? ldexpf(1.0f, -e) : 0.0f;
  for (int b = threadIdx.x; b < nb; b += kPrepThreads) {
    float v[8];
    if (scale != 0.0f) {
      load8<float>(hr, b, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    half8 h0, h1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float t = v[kCodeOrder[i]] * scale;
      const _Float16 hi = static_cast<_Float16>(t);
      h0[i] = hi;
      if (P == 2) h1[i] = static_cast<_Float16>(t - static_cast<float>(hi));
    }
    *reinterpret_cast<half8*>(ap + static_cast<size_t>(row) * I + 8 * b) = h0;
    if (P == 2) *reinterpret_cast<half8*>(ap + (static_cast<size_t>(Mp) + row) * I + 8 * b) = h1;
  }
}

// The pieces of h per K split of the down projection, from the gate/up
// split planes.  Workgroup (row, c) takes the h columns [c * cols, (c + 1) *
// cols) of one row, which down split c reads: it sums the gate/up planes in
// split order, forms h = silu(g * f) * (u * f) in registers, and scales the
// pieces to the largest magnitude of that range alone (as mfma_prep_kernel
// does for a whole row): rs[c * Mp + row] = 2^-e_c.  Down split c then sums
// in units of 2^-e_c, which the plane sum multiplies back before it adds the
// splits.  Each thread keeps up to kSplitPrepBlocks blocks of 8 values;
// rows M .. Mp-1 get zero pieces and rs 0.
constexpr int kSplitPrepThreads = 256;
constexpr int kSplitPrepBlocks = 4;
constexpr int kSplitPrepBatch = 4;  // gate/up split planes read together

template <int P>
__global__ __launch_bounds__(kSplitPrepThreads) void prep_split_pieces_kernel(
    const float* __restrict__ planes, int S, int plane_rows, int plane_ld, const float* __restrict__ rsx, int M,
    int Mp, int I, int cols, _Float16* __restrict__ ap, float* __restrict__ rs) {
  __shared__ float red[kSplitPrepThreads / kWave];
  const int row = blockIdx.x, c = blockIdx.y;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int n0 = c * cols;
  const int nbc = min(cols, I - n0) / 8;
  float v[kSplitPrepBlocks][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kSplitPrepBlocks; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) v[i][j] = 0.0f;
  if (row < M) {
    const float f = rsx[row];
    const size_t sstride = static_cast<size_t>(2) * plane_rows * plane_ld;  // one split: gate plane + up plane
    const float* gp = planes + static_cast<size_t>(row) * plane_ld + n0;
    const float* up = gp + static_cast<size_t>(plane_rows) * plane_ld;
#pragma unroll
    for (int i = 0; i < kSplitPrepBlocks; ++i) {
      const int b = tid + i * nt;
      if (b < nbc) {
        f32x4 g0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, g1 = g0, u0 = g0, u1 = g0;
        // kSplitPrepBatch splits' loads in flight together, summed in split order
        for (int s0 = 0; s0 < S; s0 += kSplitPrepBatch) {
          f32x4 q[kSplitPrepBatch][4];
#pragma unroll
          for (int j = 0; j < kSplitPrepBatch; ++j)
            if (s0 + j < S) {
              const size_t o = (s0 + j) * sstride + 8 * static_cast<size_t>(b);
              q[j][0] = *reinterpret_cast<const f32x4*>(gp + o);
              q[j][1] = *reinterpret_cast<const f32x4*>(gp + o + 4);
              q[j][2] = *reinterpret_cast<const f32x4*>(up + o);
              q[j][3] = *reinterpret_cast<const f32x4*>(up + o + 4);
            }
#pragma unroll
          for (int j = 0; j < kSplitPrepBatch; ++j)
            if (s0 + j < S) {
              g0 += q[j][0];
              g1 += q[j][1];
              u0 += q[j][2];
              u1 += q[j][3];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[i][j] = silu(g0[j] * f) * (u0[j] * f);
          v[i][4 + j] = silu(g1[j] * f) * (u1[j] * f);
          amax = fmaxf(amax, fmaxf(fabsf(v[i][j]), fabsf(v[i][4 + j])));
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (lane_id() == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = 0.0f;
  for (int w = 0; w < nt / kWave; ++w) amax = fmaxf(amax, red[w]);
  int e = 0;
  if (amax > 0.0f) {
    int lg = ilogbf(amax);
    lg = lg > 120 ? 120 : (lg < -120 ? -120 : lg);
    e = 14 - lg;
  }
  const float scale = amax > 0.0f ? ldexpf(1.0f, e) : 0.0f;
  if (tid == 0) rs[static_cast<size_t>(c) * Mp + row] = scale > 0.0f ? ldexpf(1.0f, -e) : 0.0f;
#pragma unroll
  for (int i = 0; i < kSplitPrepBlocks; ++i) {
    const int b = tid + i * nt;
    if (b < nbc) {
      half8 h0, h1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = scale != 0.0f ? v[i][kCodeOrder[j]] * scale : 0.0f;
        const _Float16 hi = static_cast<_Float16>(t);
        h0[j] = hi;
        if (P == 2) h1[j] = static_cast<_Float16>(t - static_cast<float>(hi));
      }
      _Float16* dst = ap + static_cast<size_t>(row) * I + n0 + 8 * b;
      *reinterpret_cast<half8*>(dst) = h0;
      if (P == 2) *reinterpret_cast<half8*>(dst + static_cast<size_t>(Mp) * I) = h1;
    }
  }
}

}  // namespace

w4a16_status_t launch_plane_sum(const float* planes, int S, int plane_rows, int plane_ld, const float* rs,
                                int rs_stride, int M, int N, float* out, hipStream_t stream, hipEvent_t start,
                                hipEvent_t stop) {
  if (M == 0 || N == 0) return W4A16_OK;
  if (S < 1 || S > kMaxSplits || N % 4 != 0 || plane_ld < N || plane_rows < M || rs_stride < 0 ||
      (rs_stride > 0 && rs_stride < M))
    return W4A16_ERR_INVALID_ARG;
  const size_t n = static_cast<size_t>(M) * (N / 4);
  const size_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  hipExtLaunchKernelGGL(plane_sum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, start, stop,
                        0, planes, S, plane_rows, plane_ld, rs, rs_stride, M, N, out);
  return launch_status();
}

// One block of 8 per thread where the range allows (more loads in flight),
// up to kSplitPrepBlocks per thread of a full workgroup.
int split_pieces_threads(int cols) {
  const int nb = cols / 8;
  if (nb > kSplitPrepThreads * kSplitPrepBlocks) return 0;
  const int t = (nb + kWave - 1) / kWave * kWave;
  return t < kWave ? kWave : (t > kSplitPrepThreads ? kSplitPrepThreads : t);
}

w4a16_status_t launch_prep_split_pieces(const float* planes, int S, int plane_rows, int plane_ld, const float* rsx,
                                        int M, int Mp, int I, int P, int cols, _Float16* ap, float* rs,
                                        hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (Mp == 0 || I == 0) return W4A16_OK;
  if (S < 1 || cols <= 0 || cols % 8 != 0 || I % 8 != 0 || plane_ld < I || plane_rows < M || Mp < M)
    return W4A16_ERR_INVALID_ARG;
  const int nt = split_pieces_threads(cols);
  if (nt == 0) return W4A16_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(Mp), static_cast<unsigned>((I + cols - 1) / cols));
  if (P == 2)
    hipExtLaunchKernelGGL(prep_split_pieces_kernel<2>, grid, dim3(nt), 0, stream, start, stop, 0, planes, S,
                          plane_rows, plane_ld, rsx, M, Mp, I, cols, ap, rs);
  else
    hipExtLaunchKernelGGL(prep_split_pieces_kernel<1>, grid, dim3(nt), 0, stream, start, stop, 0, planes, S,
                          plane_rows, plane_ld, rsx, M, Mp, I, cols, ap, rs);
  return launch_status();
}

w4a16_status_t launch_prep_planes(const float* planes, int S, int plane_rows, int plane_ld, const float* rsx,
                                  int M, int Mp, int I, int P, float* h, _Float16* ap, float* rs,
                                  hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (Mp == 0) return W4A16_OK;
  if (S < 1 || I % 8 != 0 || plane_ld < I || plane_rows < M || Mp < M) return W4A16_ERR_INVALID_ARG;
  if (P == 2)
    hipExtLaunchKernelGGL(prep_planes_kernel<2>, dim3(Mp), dim3(kPrepThreads), 0, stream, start, stop, 0, planes,
                          S, plane_rows, plane_ld, rsx, M, Mp, I, h, ap, rs);
  else
    hipExtLaunchKernelGGL(prep_planes_kernel<1>, dim3(Mp), dim3(kPrepThreads), 0, stream, start, stop, 0, planes,
                          S, plane_rows, plane_ld, rsx, M, Mp, I, h, ap, rs);
  return launch_status();
}

w4a16_status_t launch_mfma_prep(const void* x, w4a16_dtype_t xt, int R, int Mp, int K, int P,
                                const int* gather, int top_k, const int* need, _Float16* ap,
                                float* rs, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (Mp == 0) return W4A16_OK;
  if (kPrepWave && K / 8 <= kWave * 4) {
    launch_prep_wave<4>(x, xt, R, Mp, K, P, gather, top_k, need, ap, rs, stream, start, stop);
    return launch_status();
  }
  if (kPrepWave && K / 8 <= kWave * 8) {
    launch_prep_wave<8>(x, xt, R, Mp, K, P, gather, top_k, need, ap, rs, stream, start, stop);
    return launch_status();
  }
  const float* xf = static_cast<const float*>(x);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const dim3 g(Mp), b(kPrepThreads);
  if (xt == W4A16_F32 && P == 2)
    hipExtLaunchKernelGGL(mfma_prep_kernel<float, 2>, g, b, 0, stream, start, stop, 0, xf, R, Mp, K, gather,
                          top_k, need, ap, rs);
  else if (xt == W4A16_F32)
    hipExtLaunchKernelGGL(mfma_prep_kernel<float, 1>, g, b, 0, stream, start, stop, 0, xf, R, Mp, K, gather,
                          top_k, need, ap, rs);
  else if (P == 2)
    hipExtLaunchKernelGGL(mfma_prep_kernel<uint16_t, 2>, g, b, 0, stream, start, stop, 0, xb, R, Mp, K, gather,
                          top_k, need, ap, rs);
  else
    hipExtLaunchKernelGGL(mfma_prep_kernel<uint16_t, 1>, g, b, 0, stream, start, stop, 0, xb, R, Mp, K, gather,
                          top_k, need, ap, rs);
  return launch_status();
}

namespace {
void launch_one_piece(const MfmaArgs& a, unsigned grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (a.dense_rows > 0 && a.planes != nullptr && a.S > 1)
    hipExtLaunchKernelGGL((mfma_kernel<1, kTileRing, 2, true>), dim3(grid), dim3(kMfmaThreads), 0, stream, start,
                          stop, 0, a);
  else if (a.dense_rows > 0)
    hipExtLaunchKernelGGL(mfma_kernel<1, kTileRing, 2>, dim3(grid), dim3(kMfmaThreads), 0, stream, start, stop,
                          0, a);
  else
    hipExtLaunchKernelGGL(mfma_kernel<1, kGroupedRing, 3>, dim3(grid), dim3(kMfmaThreads), 0, stream, start,
                          stop, 0, a);
}
}  // namespace

w4a16_status_t launch_mfma(const MfmaArgs& a, int P, size_t num_tasks, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
  if (num_tasks == 0) return W4A16_OK;
  if (num_tasks > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  // a split's codes must stay within the kernel's 32-bit buffer offsets
  if (static_cast<size_t>(a.gps) * a.N * 16 > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  const unsigned grid = static_cast<unsigned>(num_tasks);
  if (a.planes != nullptr && a.S > 1 && a.dense_rows <= 0) return W4A16_ERR_INVALID_ARG;  // dense rows only
  if (P == 2 && a.planes != nullptr && a.S > 1)
    hipExtLaunchKernelGGL((mfma_kernel<2, kTileRing, 2, true>), dim3(grid), dim3(kMfmaThreads), 0, stream, start,
                          stop, 0, a);
  else if (P == 2)
    hipExtLaunchKernelGGL(mfma_kernel<2, kTileRing, 2>, dim3(grid), dim3(kMfmaThreads), 0, stream, start, stop,
                          0, a);
  else
    launch_one_piece(a, grid, stream, start, stop);
  return launch_status();
}

}  // namespace w4
