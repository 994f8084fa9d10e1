// Wide MFMA tiles for large row counts with bf16 activations.
//
// y[m][n] = sum_g s[g][n] * sum_{k in g} x[m][k] * q[k][n]   (page "The Weight
// of Precision: Building Native INT4 Quantization for a Custom Speculative
// Decoding Engine", section "The Kernel: w4a16_gemm").
//
// The operands are those of the 64-row tile kernel's one-piece mode: A is the
// f16 piece of x * 2^e per row (mfma.h), B the weights expanded to
// f16(q * f16(s * 2^c)), accumulated by v_mfma_f32_16x16x32_f16 in float32 and
// brought back by 2^-c per column and 2^-e per row at the end.  Here c is fixed
// per column for the whole launch: the workgroup first reads the column's
// scales over all of K and puts the largest in [1/2, 1), so no product can
// leave the f16 range and no accumulator ever needs rescaling.
//
// A workgroup computes 256 rows x 128 columns with eight waves, two per SIMD:
// wave (kh, wr, wc) = (wv >> 2, (wv >> 1) & 1, wv & 1) owns rows 128wr ..
// +127 and columns 64wc .. +63, and the K half kh: of each window's four
// groups it takes groups kh and kh + 2.  Per group a wave runs 8 x 4 MFMA
// blocks of 16 x 16, so every expanded weight feeds 8 MFMAs, twice the 64-row
// tile's reuse, and the vector work per matrix-core instruction halves.  The
// 256 x 128 activation window (four groups, 64 KiB) is staged once in LDS,
// double-buffered, with one workgroup barrier per window; each wave streams
// its own 64 columns of codes of its own groups, one 16-byte GROUPED slot per
// lane and group.  After the loop the second K half's sums are added to the
// first half's through LDS, in that order.  (With one wave per SIMD and every
// wave on both groups of a two-group window, the 2048 x 7168 x 4096 GEMM took
// 138-142 us here; with two-group windows, a barrier every two groups,
// 129-132 against 125-127 us.)
//
// Workgroups are numbered so that each XCD (the hardware deals workgroup b to
// XCD b mod 8) takes a contiguous run of tiles, row tile major: the column
// tiles of one row tile then share that XCD's L2 for their activations.
#include <type_traits>

#include "mfma.h"
#include "mfma_ops.h"

#include <hip/hip_ext.h>

namespace w4 {
namespace {

constexpr int kWw = 4;                                     // groups per staged activation window (two per K half)
constexpr int kWideWgThreads = 2 * kWideThreads;           // two K halves of four waves
constexpr int kWideRing = 2;                               // own groups of codes in flight per wave (two windows)
constexpr int kWideWinUnits = kWw * kWideRows * 4;         // 16-byte units per window
constexpr int kWideUnitsPerThread = kWideWinUnits / kWideWgThreads;
constexpr int kAnchorBatch = 8;                            // scale loads in flight per thread
constexpr int kAnchorPhases = kWideWgThreads / 32;         // scale rows read at once (32 column quads)
constexpr int kXcds = 8;
constexpr int kAhead = 1;                                  // A fragments read ahead of their MFMAs

// Raw buffer resources: a wave-uniform base and size in scalar registers, so a
// load takes one 32-bit lane offset and a scalar offset (no 64-bit address
// arithmetic per load).  The size check covers the lane offset only, not the
// scalar one, so every scalar offset below is kept inside its buffer.
constexpr int kBufFlags = 0x00020000;  // dword 3 of a raw buffer resource on gfx9

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = bytes >= 0x7fffffffu ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kBufFlags);
}

// Unit (gl, row, kb) of a window: the four 16-byte k blocks of a row are
// permuted by a 2-bit function of the row so that the 8 (or 16) lanes one LDS
// cycle serves, rows r .. r+7 (r .. r+15) of one k block for an A fragment
// read, fall in distinct 16-byte bank groups whether the LDS has 32 or 64
// banks; the staging stores (two rows x four k blocks per 8 lanes) are
// conflict-free with any such permutation.
__device__ __forceinline__ int a_swz(int row) { return (((row >> 1) ^ (row >> 3)) & 1) | ((row >> 1) & 2); }
__device__ __forceinline__ int w_off(int gl, int row, int kb) {
  return (gl * kWideRows + row) * 4 + (kb ^ a_swz(row));
}

struct WideLds {
  uint4 a[2][kWideWinUnits];  // double buffer, 2 x 64 KiB
  float red[kAnchorPhases][kWideCols];  // anchor reduction
  int cexp[kWideCols];
  int last;
};

// Staging: thread t handles units u = t + 512 i, k block u & 3, row
// 8 (u >> 6) + ((u >> 2) & 7), group (u >> 5) & 1: each 8 lanes two rows of
// one group, each wave 8 rows x both groups.  The lane offset holds t's row,
// group and k block; the scalar offset the window's first group and 64 i
// rows.  The prefetch after a split's last window reads the next split's
// activations, or past the end of the row (at most 128 bytes past the last
// row of the plane, which the workspace pads), and is never used.
__device__ __forceinline__ int stage_row(int u) { return 8 * (u >> 6) + ((u >> 2) & 7); }

// A window is staged in four parts of kPartUnits units per thread, so that
// only one part is held in registers at a time.  Unit i of a thread covers
// rows + 64 (i & 3) of the groups pair i >> 2 (window groups 0-1 or 2-3).
constexpr int kParts = 4;
constexpr int kPartUnits = kWideUnitsPerThread / kParts;
__device__ __forceinline__ void wide_load_a(__amdgpu_buffer_rsrc_t ra_src, int voff, int K, int gw, int part,
                                            uint4 r[kPartUnits]) {
#pragma unroll
  for (int j = 0; j < kPartUnits; ++j) {
    const int i = part * kPartUnits + j;
    r[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                         ra_src, voff, ((gw + 2 * (i >> 2)) * kGroup + 64 * (i & 3) * K) * 2, 0));
  }
}

// Every split holds a multiple of four groups (the launch checks it), so a
// window is always whole.
__device__ __forceinline__ void wide_store_a(uint4* buf, int part, const uint4 r[kPartUnits]) {
#pragma unroll
  for (int j = 0; j < kPartUnits; ++j) {
    const int i = part * kPartUnits + j;
    const int u = static_cast<int>(threadIdx.x) + kWideWgThreads * (i & 3);
    buf[w_off(((u >> 5) & 1) + 2 * (i >> 2), stage_row(u), u & 3)] = r[j];
  }
}

struct WideCodes {
  u32x4 w;  // word kb of the lane's four columns
  f32x4 s;  // their scales
};

// Codes and scales of group g (wave-uniform): the lane offsets are fixed, the
// group moves the scalar offset.  Prefetches past the matrix's last group
// re-read that group.
__device__ __forceinline__ void wide_load_codes(__amdgpu_buffer_rsrc_t wsrc, __amdgpu_buffer_rsrc_t ssrc, int wvoff,
                                                int svoff, int N, int g_req, int g_max, int gshift, WideCodes& c) {
  const int g = min(g_req, g_max);
  c.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wsrc, wvoff, g * N * 16, 0));
  c.s = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ssrc, svoff, (g >> gshift) * N * 4, 0));
}

// The matrix-core step with the accumulator tied in place (the compiler's
// own form writes a fresh register and copies it back every loop trip).
// Being opaque to the compiler, it gets no hazard padding: every use below
// keeps its operands' producers and consumers well apart, and the kernel
// pads the accumulators' first write and last read itself.
__device__ __forceinline__ void mfma_tied(f32x4& acc, const half8& a, const half8& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Expansion of one code word and its anchored scale into
// f16(q * f16(s * 2^c)), k order 0,4,1,5,2,6,3,7 (the A pieces' order), cut
// into eight steps of one or two vector instructions that the main loop
// spreads between its MFMAs.  A nibble under an f16 exponent of 0x6400 reads
// as 1024 + n (bits 0..3) or 1024 + 16 n (bits 4..7): one packed subtract of
// 1032, or one packed fma (x / 16 - 72), leaves n - 8 exactly.
struct WordExp {
  half2v h, p0, p1, p2, p3;
  uint32_t hi;
};

template <int kStep>
__device__ __forceinline__ void expand_step(uint32_t w, float s, int ce, uint32_t magic, WordExp& e, half8& out) {
  const half2v sub = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const half2v sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const half2v off = {static_cast<_Float16>(-72.0f), static_cast<_Float16>(-72.0f)};
  if constexpr (kStep == 0) {
    const _Float16 hh = static_cast<_Float16>(ldexpf(s, ce));
    e.h = half2v{hh, hh};
  } else if constexpr (kStep == 1) {
    e.p0 = __builtin_bit_cast(half2v, (w & 0x000f000fu) | magic) + sub;
  } else if constexpr (kStep == 2) {
    e.p1 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, (w & 0x00f000f0u) | magic), sixteenth, off);
  } else if constexpr (kStep == 3) {
    e.hi = w >> 8;
    e.p2 = __builtin_bit_cast(half2v, (e.hi & 0x000f000fu) | magic) + sub;
  } else if constexpr (kStep == 4) {
    e.p3 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, (e.hi & 0x00f000f0u) | magic), sixteenth, off);
  } else if constexpr (kStep == 5) {
    e.p0 = e.p0 * e.h;
    e.p1 = e.p1 * e.h;
  } else if constexpr (kStep == 6) {
    e.p2 = e.p2 * e.h;
    e.p3 = e.p3 * e.h;
  } else {
    out = half8{e.p0[0], e.p0[1], e.p1[0], e.p1[1], e.p2[0], e.p2[1], e.p3[0], e.p3[1]};
  }
}

__global__ __launch_bounds__(kWideWgThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void wide_kernel(const MfmaArgs a) {
  __shared__ WideLds lds;
  const int t = static_cast<int>(threadIdx.x);

  // XCD-aware task order: XCD x = b mod 8 takes tasks x*q + min(x, r) + b / 8
  // of T = 8q + r, a bijection onto 0 .. T-1 for b < T.
  const int T = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int xcd = b % kXcds, q = T / kXcds, rem = T % kXcds;
  const int task = xcd * q + min(xcd, rem) + b / kXcds;
  const int split = task % a.S;
  const int rest = task / a.S;
  const int tile = rest % a.tiles;
  const int item = rest / a.tiles;
  const int row0 = item * kWideRows;

  const int wv = __builtin_amdgcn_readfirstlane(wave_id());
  const int lane = lane_id();
  const int lc = lane & 15, kb = lane >> 4;
  const int kh = wv >> 2, wr = (wv >> 1) & 1, wc = wv & 1;  // K half, row half, column half
  const uint32_t magic = magic_vgpr();

  const int c0 = tile * kWideCols + wc * 64;
  const bool wave_ok = c0 < a.N;
  const int col0 = c0 + 4 * lc;
  const __amdgpu_buffer_rsrc_t wsrc = make_rsrc(a.qw0, static_cast<size_t>(a.G) * a.N * 16);
  const __amdgpu_buffer_rsrc_t ssrc = make_rsrc(a.sc0, static_cast<size_t>(a.G >> a.gshift) * a.N * 4);
  const int wvoff = ((wave_ok ? c0 : 0) + 16 * kb + lc) * 16;
  const int svoff = (wave_ok ? col0 : 4 * lc) * 4;
  const __amdgpu_buffer_rsrc_t asrc =
      make_rsrc(a.ap + static_cast<size_t>(row0) * a.K, static_cast<size_t>(kWideRows) * a.K * 2);
  const int avoff = (stage_row(t) * a.K + ((t >> 5) & 1) * kGroup + 8 * (t & 3)) * 2;  // unit t of the staging map

  const int g_lo = split * a.gps;
  const int g_hi = min(a.G, g_lo + a.gps);
  const int nwin = (g_hi - g_lo + kWw - 1) / kWw;
  // this wave's own groups: g_lo + kh + 2 j, two per window (window groups kh
  // and kh + 2)
  auto own = [&](int j) { return g_lo + kh + 2 * j; };

  uint4 ra[kPartUnits];
  WideCodes ring[kWideRing];  // own group j sits in slot j % kWideRing
  wide_load_a(asrc, avoff, a.K, g_lo, 0, ra);
#pragma unroll
  for (int j = 0; j < kWideRing; ++j) {
    wide_load_codes(wsrc, ssrc, wvoff, svoff, a.N, own(j), a.G - 1, a.gshift, ring[j]);
    __builtin_amdgcn_sched_barrier(0);  // issue order = use order
  }

  // Column anchors over every scale row of K: thread t reads columns
  // 4(t & 31) .. +3 of the tile at scale rows t >> 5, + 16, ... (rows past the
  // end are clamped to the last one; a repeated row leaves a maximum as it is).
  {
    const int cq = t & 31, r0 = t >> 5;
    const int ccol = tile * kWideCols + 4 * cq;
    const int ccl = ccol < a.N ? ccol : 0;
    const int rows = a.G >> a.gshift;
    f32x4 mx = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int r = r0; r < rows; r += kAnchorPhases * kAnchorBatch) {
      f32x4 v[kAnchorBatch];
#pragma unroll
      for (int j = 0; j < kAnchorBatch; ++j)
        v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             ssrc, (min(r + kAnchorPhases * j, rows - 1) * a.N + ccl) * 4, 0, 0));
#pragma unroll
      for (int j = 0; j < kAnchorBatch; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx[e] = fmaxf(mx[e], fabsf(v[j][e]));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) lds.red[r0][4 * cq + e] = mx[e];
    __syncthreads();
    if (t < kWideCols) {
      float m = lds.red[0][t];
#pragma unroll
      for (int j = 1; j < kAnchorPhases; ++j) m = fmaxf(m, lds.red[j][t]);
      lds.cexp[t] = m > 0.0f ? -__builtin_amdgcn_frexp_expf(m) : 0;
    }
  }
  wide_store_a(lds.a[0], 0, ra);
#pragma unroll
  for (int part = 1; part < kParts; ++part) {
    wide_load_a(asrc, avoff, a.K, g_lo, part, ra);
    wide_store_a(lds.a[0], part, ra);
  }
  __syncthreads();
  int cexp[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) cexp[cb] = lds.cexp[wc * 64 + 4 * lc + cb];

  f32x4 acc[8][4];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Window wi uses LDS buffer h = wi % 2 and holds this wave's own groups
  // 2 wi and 2 wi + 1 (own group j sits in ring slot j % 2); the loop body is
  // two whole windows and an odd last window runs after it, so every path into
  // the loop header has the same loads outstanding.  An own group is a pass
  // of 8 row-block steps, each one A fragment read (kAhead steps ahead) and 4
  // MFMAs; between the MFMAs run the steps of the expansion of the wave's
  // next own group, whose slot is then refilled with own group j + 1 +
  // kWideRing.  The schedule is pinned with scheduling barriers.
  half8 bq[2][4];  // expanded weights, by own-group parity
  {
    WordExp e;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      expand_step<0>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
      expand_step<1>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
      expand_step<2>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
      expand_step<3>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
      expand_step<4>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
      expand_step<5>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
      expand_step<6>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
      expand_step<7>(ring[0].w[cb], ring[0].s[cb], cexp[cb], magic, e, bq[0][cb]);
    }
  }
  wide_load_codes(wsrc, ssrc, wvoff, svoff, a.N, own(kWideRing), a.G - 1, a.gshift, ring[0]);
  // the accumulators were just written by vector instructions: pad before
  // the first (opaque) MFMA reads them
  asm volatile("s_nop 7\n\ts_nop 7");
  auto window = [&](int wi, auto hc) {
    constexpr int h = decltype(hc)::value;
    const int gw = g_lo + wi * kWw;
    wide_load_a(asrc, avoff, a.K, gw + kWw, 0, ra);  // part 0 of the next window, in flight
    const uint4* buf = lds.a[h];
    static_assert(2 % kWideRing == 0, "ring slots repeat with the two passes of a window");
    // Pass p computes this wave's own group 2 wi + p (window group kh + 2 p).
    // The next window's parts are stored (buffer 1 - h is free) and fetched
    // at rb = 4 of pass 0, rb = 0 and rb = 4 of pass 1, and after pass 1.
    auto pass = [&](auto pc) {
      constexpr int p = decltype(pc)::value;
      auto rd = [&](int st) {
        return __builtin_bit_cast(half8, buf[w_off(kh + 2 * p, wr * 128 + st * 16 + lc, kb)]);
      };
      half8 af[4];
#pragma unroll
      for (int st = 0; st < kAhead; ++st) af[st] = rd(st);
      __builtin_amdgcn_sched_barrier(0);
      constexpr int cur = p;                      // this own group's expanded weights
      constexpr int nslot = (p + 1) % kWideRing;  // ring slot of the next own group
      WordExp e;
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        if (p == 1 && rb == 0) {
          wide_store_a(lds.a[1 - h], 1, ra);
          wide_load_a(asrc, avoff, a.K, gw + kWw, 2, ra);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (rb == 4) {
          wide_store_a(lds.a[1 - h], 2 * p, ra);
          wide_load_a(asrc, avoff, a.K, gw + kWw, 2 * p + 1, ra);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (rb + kAhead < 8) af[(rb + kAhead) & 3] = rd(rb + kAhead);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          mfma_tied(acc[rb][cb], af[rb & 3], bq[cur][cb]);
          // expansion step (rb * 4 + cb) % 8 of word (rb * 4 + cb) / 8
          const int x = rb * 4 + cb, word = x >> 3;
          const uint32_t wd = ring[nslot].w[word];
          const float sc = ring[nslot].s[word];
          half8& o = bq[cur ^ 1][word];
          switch (x & 7) {
            case 0: expand_step<0>(wd, sc, cexp[word], magic, e, o); break;
            case 1: expand_step<1>(wd, sc, cexp[word], magic, e, o); break;
            case 2: expand_step<2>(wd, sc, cexp[word], magic, e, o); break;
            case 3: expand_step<3>(wd, sc, cexp[word], magic, e, o); break;
            case 4: expand_step<4>(wd, sc, cexp[word], magic, e, o); break;
            case 5: expand_step<5>(wd, sc, cexp[word], magic, e, o); break;
            case 6: expand_step<6>(wd, sc, cexp[word], magic, e, o); break;
            default: expand_step<7>(wd, sc, cexp[word], magic, e, o); break;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      wide_load_codes(wsrc, ssrc, wvoff, svoff, a.N, own(2 * wi + p + 1 + kWideRing), a.G - 1, a.gshift,
                      ring[nslot]);
      __builtin_amdgcn_sched_barrier(0);
    };
    pass(std::integral_constant<int, 0>{});
    pass(std::integral_constant<int, 1>{});
    wide_store_a(lds.a[1 - h], 3, ra);
    __syncthreads();
  };
  int w = 0;
  for (; w + 1 < nwin; w += 2) {
    window(w, std::integral_constant<int, 0>{});
    window(w + 1, std::integral_constant<int, 1>{});
  }
  if (w < nwin) window(w, std::integral_constant<int, 0>{});
  // the last (opaque) MFMAs' results are read by vector instructions below
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");

  // The two K halves meet in LDS (the window buffers are free after the loop's
  // last barrier), one row half at a time: the second half's waves store
  // their sums, the first half's add them, in that order.
  {
    float* red = reinterpret_cast<float*>(&lds.a[0][0]);
    static_assert(sizeof(lds.a) >= 2 * 128 * 64 * sizeof(float), "a row half of sums must fit in the windows");
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (kh == 1 && wr == p) {
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[((wc * 128 + (rb * 4 + cb) * 4 + i) << 6) + lane] = acc[rb][cb][i];
      }
      __syncthreads();
      if (kh == 0 && wr == p) {
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
          for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rb][cb][i] += red[((wc * 128 + (rb * 4 + cb) * 4 + i) << 6) + lane];
      }
      __syncthreads();
    }
  }

  // Split-K across workgroups (first K half's threads t < kWideThreads hold
  // the tile): write-through partials [j][thread], j = (rb * 4 + cb) * 4 + i,
  // an agent-scope arrival counter, and the last workgroup sums the partials
  // in split order, 32 loads per thread in flight (the GEMV kernel's scheme
  // and its reliance on gfx950's write-through agent-scope atomics).  Every
  // thread reaches the barriers.
  if (a.S > 1) {
    const size_t ct = static_cast<size_t>(item) * a.tiles + tile;
    const size_t tf = static_cast<size_t>(kWideRows) * kWideCols;
    float* base = a.partials + ct * a.S * tf + (kh == 0 ? t : 0);
    if (kh == 0) {
#pragma unroll
      for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __hip_atomic_store(base + split * tf + ((rb * 4 + cb) * 4 + i) * kWideThreads, acc[rb][cb][i],
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
    __syncthreads();
    if (t == 0)
      lds.last = (__hip_atomic_fetch_add(&a.counters[ct], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  a.S - 1);
    __syncthreads();
    if (!lds.last || kh != 0) return;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < a.S; ++s) {
      const float* ps = base + static_cast<size_t>(s) * tf;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        float p[32];
#pragma unroll
        for (int e = 0; e < 32; ++e)
          p[e] = __hip_atomic_load(ps + (hh * 32 + e) * kWideThreads, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int j = hh * 32 + e;
          acc[j >> 4][(j >> 2) & 3][j & 3] += p[e];
        }
      }
    }
    if (t == 0) __hip_atomic_store(&a.counters[ct], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!wave_ok || kh != 0) return;

  // lane (lc, kb) holds rows rb*16 + 4kb + i of columns col0 .. col0 + 3 (the
  // four column blocks): one 16-byte store per row
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + wr * 128 + rb * 16 + 4 * kb + i;
      if (r < a.dense_rows) {
        const float f = a.rs[r];
        float4 o;
        o.x = ldexpf(acc[rb][0][i], -cexp[0]) * f;
        o.y = ldexpf(acc[rb][1][i], -cexp[1]) * f;
        o.z = ldexpf(acc[rb][2][i], -cexp[2]) * f;
        o.w = ldexpf(acc[rb][3][i], -cexp[3]) * f;
        *reinterpret_cast<float4*>(a.out + static_cast<size_t>(r) * a.N + col0) = o;
      }
    }
}

}  // namespace

w4a16_status_t launch_wide(const MfmaArgs& a, size_t num_tasks, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
  if (num_tasks == 0) return W4A16_OK;
  if (num_tasks > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  if (a.mode != 0 || a.dense_rows <= 0 || a.Mp % kWideRows != 0 || a.G % kWw != 0 || a.gps % kWw != 0)
    return W4A16_ERR_UNSUPPORTED;
  hipExtLaunchKernelGGL(wide_kernel, dim3(static_cast<unsigned>(num_tasks)), dim3(kWideWgThreads), 0, stream, start,
                        stop, 0, a);
  return launch_status();
}

}  // namespace w4
