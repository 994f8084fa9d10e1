// Split-K W4A16 GEMV on the matrix cores for decode-sized row counts.
//
// y[m][n] = sum_g s[g][n] * sum_{k in g} x[m][k] * q[k][n]   (page "The Weight
// of Precision: Building Native INT4 Quantization for a Custom Speculative
// Decoding Engine", section "The Kernel: w4a16_gemm": per-group scales on
// symmetric INT4 codes).
//
// A task covers up to eight rows.  One v_mfma_f32_16x16x32_f16 spans exactly
// one 32-row scale group and 16 weight columns: its B operand holds the exact
// codes (codes_f16), its 16 A rows the two f16 pieces of the rescaled
// activations of the eight rows (A rows 0..7: piece 0, rows 8..15: piece 1).
// Each group's 16x16 result is scaled by s[g][n] on float32 accumulators and
// the two pieces are added once at the end.  The vector work per 16 columns
// and group (nine instructions of code expansion, four scale fmas) does not
// depend on the row count, so the kernel streams the weights at memory speed
// from one row to eight.
//
// A workgroup owns 256 weight columns (a 64-column block per wave; in SwiGLU
// mode 128 gate and the same 128 up columns) and one K split.  A lane reads
// one 16-byte GROUPED slot and one 16-byte run of scales per group: the codes
// of four adjacent columns for one 8-row block, which are column lc of the
// four MFMA blocks.  The activations of the split
// are staged in LDS one window of groups at a time, with one power-of-two
// rescale per row and window (the row's largest magnitude maps into
// [2^14, 2^15), so f16 neither overflows nor loses the large values); each
// window's accumulators are scaled back by 2^-e before they join the total.
#include "gemv.h"

#include <hip/hip_ext.h>
#include "mfma_ops.h"

namespace w4 {
namespace {

#ifndef W4_GEMV_PACE
#define W4_GEMV_PACE 1
#endif
constexpr int kPace = W4_GEMV_PACE;      // ring rounds between pacing barriers (0: none)
constexpr int kWin = 32;                 // groups per staging window
#ifndef W4_GEMV_RING
#define W4_GEMV_RING 4
#endif
constexpr int kRing = W4_GEMV_RING;       // groups of codes in flight per wave
constexpr int kUnitsPerGroup = 16 * 4;   // 16-byte units of one group's A (16 rows x 4 k blocks)

struct GemvLds {
  // A operand of the window, unit (g, r, kb) at a_unit(g, r, kb); reused after
  // the main loop as the tile buffers [kT][rows][kGemvCols] of floats
  uint4 buf[kWin * kUnitsPerGroup];
  float f[kGemvRowsOnePiece];  // per row: 2^(e - e before this window), the accumulators' rescale
  int e[kGemvRowsOnePiece];    // per row: the running exponent e (kNoExp before any nonzero value)
};
constexpr int kNoExp = 1 << 20;
static_assert(kWin % kRing == 0, "ring slots must stay aligned across windows");
// four quads of 8 rows, or two of 16
static_assert(sizeof(uint4) * kWin * kUnitsPerGroup >= sizeof(float) * 4 * kMaxGemvRows * kGemvCols,
              "the tile buffers of a workgroup must fit in the staging buffer");

// The low four bits of a unit's index pick one of 16 four-bank groups:
// 4 * ((r & 3) ^ (g & 3)) + (kb ^ ((r >> 2) & 3) ^ ((g >> 2) & 1)).  A fragment
// read (16 rows at one g and kb) and a staging store (16 lanes: one row,
// eight groups, two k blocks) both cover all 16.  Rows are permuted only
// within blocks of four.
__device__ __forceinline__ int a_unit(int g, int r, int kb) {
  return (g * 16 + ((r & ~3) | ((r & 3) ^ (g & 3)))) * 4 + (kb ^ ((r >> 2) & 3) ^ ((g >> 2) & 1));
}

// Staging of groups [gw, gw + nw) of rows pos0 .. pos0 + nrows - 1 (up to
// kRows) by a workgroup of kW waves.  Wave wv takes rows wv + j * kRowStride
// (waves past kRowStride stage nothing), at most kHold rows at a time in
// registers, in kPasses passes; lane l takes 16 consecutive activations of a
// row: group l >> 1, k blocks 2(l & 1) and 2(l & 1) + 1.  The raw loads are
// split from the conversion so the first pass can be issued ahead of the
// weight prefetch (vector loads complete in order).
template <int kW, int kRows>
struct Staging {
  static constexpr int kRowStride = kW < kRows ? kW : kRows;
  static constexpr int kRowsPerWave = kRows / kRowStride;
  static constexpr int kHold = kRowsPerWave < 2 ? kRowsPerWave : 2;
  static constexpr int kPasses = kRowsPerWave / kHold;
};

template <int kW, int kRows>
__device__ __forceinline__ void load_window(const GemvArgs& a, int gw, int nw, int pos0, int nrows,
                                            int wv, int lane, int pass,
                                            float v[Staging<kW, kRows>::kHold][16]) {
  using St = Staging<kW, kRows>;
  const int gl = lane >> 1, hb = lane & 1;
#pragma unroll
  for (int j = 0; j < St::kHold; ++j) {
    const int m = wv + (pass * St::kHold + j) * St::kRowStride;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[j][i] = 0.0f;
    if (m >= nrows || wv >= St::kRowStride) continue;
    long src = pos0 + m;
    if (a.gather != nullptr) {
      const int pr = a.gather[pos0 + m];
      src = pr < 0 ? -1 : pr / a.top_k;
    }
    if (src < 0 || gl >= nw) continue;
    const size_t base = static_cast<size_t>(src) * a.K + static_cast<size_t>(gw + gl) * kGroup + 16 * hb;
    if (a.x_bf16) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + base);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 u = p[q];
        const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[j][8 * q + 2 * t] = __uint_as_float(wd[t] << 16);
          v[j][8 * q + 2 * t + 1] = __uint_as_float(wd[t] & 0xffff0000u);
        }
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + base);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 u = p[q];
        v[j][4 * q] = u.x;
        v[j][4 * q + 1] = u.y;
        v[j][4 * q + 2] = u.z;
        v[j][4 * q + 3] = u.w;
      }
    }
  }
}

// Per row, a running power of two 2^e over the windows of the split: e is
// the smallest of the previous e and the one that puts this window's largest
// magnitude in [2^14, 2^15), so f16 never overflows and the largest values so
// far keep full precision.  The pieces of x * 2^e go to LDS in the A layout;
// lds.f gets 2^(e - e before), by which the accumulators are rescaled before
// the window joins them (an exact power of two, at most 1), and lds.e the new
// e.  Two pieces (8 rows): piece 0 is A row m, piece 1 A row 8 + m.  One piece
// (16 rows, for bf16 activations it is exact): A row m.  Absent rows get the
// factor 0 and are never read as A.
template <int kW, int kRows, int kP>
__device__ __forceinline__ void convert_window(GemvLds& lds, int nw, int nrows, int wv, int lane, int pass,
                                               bool first, const float v[Staging<kW, kRows>::kHold][16]) {
  using St = Staging<kW, kRows>;
  const int gl = lane >> 1, hb = lane & 1;
  if (wv >= St::kRowStride) return;  // (wave-uniform) rows are staged by the first waves
#pragma unroll
  for (int j = 0; j < St::kHold; ++j) {
    const int m = wv + (pass * St::kHold + j) * St::kRowStride;
    if (m >= nrows) {
      if (lane == 0) {
        lds.f[m] = 0.0f;
        lds.e[m] = kNoExp;
      }
      continue;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    int e_win = kNoExp;
    if (amax > 0.0f) {
      int lg = ilogbf(amax);
      lg = lg > 120 ? 120 : (lg < -112 ? -112 : lg);  // 2^e stays a normal float
      e_win = 14 - lg;
    }
    const int e_old = first ? kNoExp : lds.e[m];  // (all lanes read before lane 0 writes)
    const int e = min(e_old, e_win);
    const float scale = e < kNoExp ? ldexpf(1.0f, e) : 0.0f;
    if (lane == 0) {
      lds.f[m] = e_old < kNoExp ? ldexpf(1.0f, e - e_old) : 1.0f;
      lds.e[m] = e;
    }
    if (gl < nw) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        half8 p0, p1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float t = v[j][8 * b + kCodeOrder[i]] * scale;
          const _Float16 h0 = static_cast<_Float16>(t);
          p0[i] = h0;
          if (kP == 2) p1[i] = static_cast<_Float16>(t - static_cast<float>(h0));
        }
        const int kb = 2 * hb + b;
        *reinterpret_cast<half8*>(&lds.buf[a_unit(gl, m, kb)]) = p0;
        if (kP == 2) *reinterpret_cast<half8*>(&lds.buf[a_unit(gl, 8 + m, kb)]) = p1;
      }
    }
  }
}

struct GroupCodes {
  uint32_t w[4];  // word kb of the lane's four columns (one per 16-column MFMA block)
  float s[4];     // the four columns' scales
};

// Codes and scales of group g (clamped to the split's last group, so the
// prefetch past the end re-reads a group that is still in cache instead of
// branching): the lane's 16-byte GROUPED slot and its four scales.
__device__ __forceinline__ void load_group(const u32x4* __restrict__ wp, const f32x4* __restrict__ sp,
                                           size_t gstride, int g, int g_last, int gshift, GroupCodes& c) {
  const size_t gg = static_cast<size_t>(min(g, g_last));
  const u32x4 w = __builtin_nontemporal_load(wp + gg * gstride);
  const f32x4 v = __builtin_nontemporal_load(sp + (gg >> gshift) * (gstride / 4));
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    c.w[cb] = w[cb];
    c.s[cb] = v[cb];
  }
}

__device__ __forceinline__ void mma_group(const GemvLds& lds, int gl, int lc, int kb, bool on,
                                          uint32_t magic, const GroupCodes& c, f32x4 acc[4]) {
  half8 af = *reinterpret_cast<const half8*>(&lds.buf[a_unit(gl, lc, kb)]);
  if (!on) af = half8{};
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const half8 bq = codes_f16(c.w[cb], magic);
    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bq, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[cb][i] = fmaf(c.s[cb], d[i], acc[cb][i]);
  }
}

// Sums of the S split partials of rows 0..nrows-1, column t, in split order:
// blocks of 4 rows x kB splits are loaded together (indices clamped into
// range, so no load is predicated) and then added.  Up to 20 splits take one
// round trip (the decode down projection runs 18).
template <int kB, int kRows>
__device__ __forceinline__ void read_partials(const float* base, int S, int nrows, int t, float v[kRows]) {
  constexpr size_t tf = kPartialTileFloats;
#pragma unroll
  for (int r0 = 0; r0 < kRows; r0 += 4) {
    if (r0 >= nrows) break;
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = 0; s0 < S; s0 += kB) {
      float p[4][kB];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int r = min(r0 + rr, nrows - 1);
          const int s2 = min(s0 + j, S - 1);
          p[rr][j] = __hip_atomic_load(base + s2 * tf + r * kGemvCols + t, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int j = 0; j < kB; ++j)
          if (s0 + j < S) sum[rr] += p[rr][j];
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (r0 + rr < nrows) v[r0 + rr] = sum[rr];
  }
}

// A workgroup is kT quads of four waves.  Quad q takes column tile
// tg * kT + q of one item and one K split, so the quads share the staged
// activation window and start streaming together (a later workgroup on a CU
// would wait for its activations behind the weight streams of the ones
// already running there).  A quad whose tile lies past the last one streams
// column block 0 and stores nothing.
//
// kP = 2: two f16 pieces of 8 rows per task (float32 activations); kP = 1:
// one piece of 16 rows (bf16 activations, which one f16 piece holds exactly,
// or the float32 intermediate of a bf16 layer).
template <int kT, int kP>
__global__ __launch_bounds__(kGemvThreads * kT) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_kernel(const GemvArgs a) {
  constexpr int kW = 4 * kT;  // waves
  constexpr int kRows = kP == 2 ? kMaxGemvRows : kGemvRowsOnePiece;  // rows per task
  static_assert(kT * kRows <= 4 * kMaxGemvRows, "tile buffers exceed the staging buffer");
  using St = Staging<kW, kRows>;
  __shared__ GemvLds lds;
  __shared__ int last[kT];

  const int tgs = (a.tiles + kT - 1) / kT;  // tile groups per item
  const int task = blockIdx.x;
  const int split = task % a.S;
  const int rest = task / a.S;
  const int item = rest / tgs;

  int expert = 0, pos0, nrows;
  if (a.dense_rows > 0) {
    pos0 = item * kRows;
    nrows = min(kRows, a.dense_rows - pos0);
  } else {
    if (item >= *a.n_items) return;
    const int4 it = a.items[item];
    expert = it.x;
    pos0 = it.y;
    nrows = it.z;
  }

  const int wv = wave_id();
  const int q = wv >> 2, wq = wv & 3;  // quad, wave within the quad
  const int tile = (rest % tgs) * kT + q;
  const bool tile_ok = tile < a.tiles;
  const int lane = lane_id();
  const int lc = lane & 15, kb = lane >> 4;
  // plain: wave wq owns columns tile*256 + 64wq ..; SwiGLU: waves 0, 1 the gate
  // and waves 2, 3 the up columns tile*128 + 64(wq & 1) ..
  int mat = 0, c0;
  if (a.mode == 1) {
    mat = wq >> 1;
    c0 = tile * (kGemvCols / 2) + (wq & 1) * 64;
  } else {
    c0 = tile * kGemvCols + wq * 64;
  }
  const bool wave_ok = tile_ok && c0 < a.N;
  const size_t ebase = static_cast<size_t>(expert) * a.expert_stride;
  const int g_lo = split * a.gps;
  const int g_hi = min(a.G, g_lo + a.gps);
  // the lane reads GROUPED slot 16kb + lc of the wave's 64-column block: word
  // kb of columns c0 + 4lc + cb, cb = 0..3 (MFMA block cb, column lc)
  const int cbase = wave_ok ? c0 : 0;
  const bool xe = expert + 1 == a.extra_plus1;
  const u32x4* qb = xe ? (mat ? a.qw1x : a.qw0x) : (mat ? a.qw1 : a.qw0) + ebase;
  const float* sb = xe ? (mat ? a.sc1x : a.sc0x) : (mat ? a.sc1 : a.sc0) + (ebase >> a.gshift);
  const u32x4* wp = qb + cbase + 16 * kb + lc;
  const f32x4* sp = reinterpret_cast<const f32x4*>(sb + cbase + 4 * lc);
  const size_t gstride = static_cast<size_t>(a.N);  // chunks (and scales) per group row
  const int g_last = g_hi - 1;
  const uint32_t magic = magic_vgpr();
  // A rows whose activations are absent read as zero (A row lc holds row
  // lc & 7 with two pieces, row lc with one)
  const bool arow = (kP == 2 ? (lc & 7) : lc) < nrows;

  f32x4 tot[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) tot[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // ring of kR groups in flight: group g sits in slot (g - g_lo) % kR.
  // Four-quad workgroups (the decode gate/up) take a ring of 2 and so meet
  // at a pacing barrier every 2 groups: 33.0-33.4 against 33.8-34.1 us for
  // that launch (a ring of 2 with the barrier every 2 groups made the
  // two-quad down projection slower, 23.2 against 21.3 us).
  constexpr int kR = kT >= 4 ? 2 : kRing;
  static_assert(kWin % kR == 0, "ring slots must stay aligned across windows");
  GroupCodes ring[kR];
  float xv[St::kHold][16];
  load_window<kW, kRows>(a, g_lo, min(kWin, g_hi - g_lo), pos0, nrows, wv, lane, 0, xv);  // ahead of the weights
  // A wave past the matrix's last column streams column block 0 and stores
  // nothing: the ring loads stay unconditional, so the compiler's waits can
  // count them.
#pragma unroll
  for (int j = 0; j < kR; ++j) load_group(wp, sp, gstride, g_lo + j, g_last, a.gshift, ring[j]);

  for (int gw = g_lo; gw < g_hi; gw += kWin) {
    const int nw = min(kWin, g_hi - gw);
    if (gw != g_lo) {
      __syncthreads();  // the previous window is consumed
      load_window<kW, kRows>(a, gw, nw, pos0, nrows, wv, lane, 0, xv);
    }
    convert_window<kW, kRows, kP>(lds, nw, nrows, wv, lane, 0, gw == g_lo, xv);
#pragma unroll
    for (int pass = 1; pass < St::kPasses; ++pass) {
      load_window<kW, kRows>(a, gw, nw, pos0, nrows, wv, lane, pass, xv);
      convert_window<kW, kRows, kP>(lds, nw, nrows, wv, lane, pass, gw == g_lo, xv);
    }
    __syncthreads();
    {
      // accumulator element i of this lane is A row 4kb + i: row (4kb + i) & 7
      // with two pieces, row 4kb + i with one.  Bring the accumulators to this
      // window's powers of two.
      const int r0 = kP == 2 ? 4 * (kb & 1) : 4 * kb;
      if (gw != g_lo) {
        const float4 f4 = *reinterpret_cast<const float4*>(&lds.f[r0]);
        const float fr[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) tot[cb][i] *= fr[i];
      }
      f32x4* acc = tot;
      // kWin is a multiple of kR, so slots stay aligned across windows; the
      // loads run kR groups ahead
      for (int gl = 0; gl < nw; gl += kR) {
#pragma unroll
        for (int j = 0; j < kR; ++j) {
          const bool on = gl + j < nw;
          mma_group(lds, on ? gl + j : gl, lc, kb, arow && on, magic, ring[j], acc);
          load_group(wp, sp, gstride, gw + gl + j + kR, g_last, a.gshift, ring[j]);
          // keep each refill right behind its consumer: the scheduler would
          // otherwise sink all refills to the end and drain the ring
          __builtin_amdgcn_sched_barrier(0);
        }
        // Pacing: each SIMD issues for its oldest wave first, so without a
        // barrier the quads of a workgroup finish one after another and the
        // CU's loads in flight fall off long before the end.  A bare barrier
        // (no memory fence, so no wait on the ring) keeps them in step.
        if (kT > 1 && kPace > 0 && (gl / kR) % kPace == kPace - 1) __builtin_amdgcn_s_barrier();
      }
    }
  }
  {
    // back from the running powers of two (rows that never had a nonzero
    // value, and absent rows, give 0)
    const int r0 = kP == 2 ? 4 * (kb & 1) : 4 * kb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lds.e[r0 + i];
      const float fr = e < kNoExp ? ldexpf(1.0f, -e) : 0.0f;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) tot[cb][i] *= fr;
    }
  }

  // two pieces: piece 0 (lanes 0..31) + piece 1 (lanes 32..63) of rows
  // 4kb + i; one piece: every lane holds rows 4kb + i
  float pv[4][4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[cb][i] = kP == 2 ? tot[cb][i] + __shfl_xor(tot[cb][i], 32) : tot[cb][i];
  __syncthreads();  // every wave is done with the staged activations
  float* red = reinterpret_cast<float*>(lds.buf);  // [kT][kRows][kGemvCols]
  if (kP == 1 || lane < 32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kb + i;
      if (m < nrows) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
          red[(q * kRows + m) * kGemvCols + wq * 64 + 4 * lc + cb] = pv[cb][i];
      }
    }
  }
  __syncthreads();

  // Thread t of quad tq owns column t of its tile, rows 0 .. nrows - 1.
  const int tq = static_cast<int>(threadIdx.x) / kGemvThreads;
  const int t = static_cast<int>(threadIdx.x) % kGemvThreads;
  const int ttile = (rest % tgs) * kT + tq;
  const bool ttile_ok = ttile < a.tiles;
  float* tred = red + tq * kRows * kGemvCols;
  float v[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) v[r] = r < nrows ? tred[r * kGemvCols + t] : 0.0f;

  // Every thread reaches every barrier below; a quad that is not the last
  // arriver of its tile only skips the stores.
  bool mine = ttile_ok;
  if (a.S > 1) {
    // Partials are written through to the device coherence point (agent-scope
    // stores), the arrival counter is an agent-scope atomic, and the last
    // workgroup of the tile reads the partials back with agent-scope loads,
    // many in flight at once, and sums them in split order.
    //
    // The ordering rests on how gfx950 executes these operations (the AMDGPU
    // backend's memory-model lowering), not on C++ release/acquire: every
    // value that crosses workgroups is an agent-scope atomic, so its store is
    // written through the XCD's L2 to the coherence point (sc1) and its load
    // reads from there; s_waitcnt vmcnt(0) returns only once this wave's
    // stores are acknowledged; the barrier then puts every wave's completed
    // stores before thread 0's counter atomic; and the last arriver's loads
    // are issued only after that atomic has returned.  No plain store is
    // published this way, so no L2 writeback or invalidate is needed; an
    // acquire-release counter (buffer_wbl2 + buffer_inv around the atomic)
    // measured 46 instead of 34 us for the decode gate/up launch.
    const size_t ct = static_cast<size_t>(item) * a.tiles + (ttile_ok ? ttile : 0);
    const size_t tf = kPartialTileFloats;
    float* base = a.partials + ct * a.S * tf;
    if (ttile_ok) {
#pragma unroll
      for (int r = 0; r < kRows; ++r)
        if (r < nrows)
          __hip_atomic_store(base + split * tf + r * kGemvCols + t, v[r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
    __syncthreads();
    if (t == 0) {
      last[tq] = ttile_ok ? (__hip_atomic_fetch_add(&a.counters[ct], 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT) == a.S - 1)
                          : 0;
    }
    __syncthreads();
    mine = last[tq] != 0;
    if (kT == 1 && !mine) return;  // a one-quad workgroup has no other quad to wait for
    if (mine) {
      if (a.S <= 8)
        read_partials<8, kRows>(base, a.S, nrows, t, v);
      else if (a.S <= 20)
        read_partials<20, kRows>(base, a.S, nrows, t, v);
      else
        read_partials<16, kRows>(base, a.S, nrows, t, v);
      if (t == 0)
        __hip_atomic_store(&a.counters[ct], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  if (a.mode == 0) {
    const int n = ttile * kGemvCols + t;
    if (mine && n < a.N) {
      uint16_t* ob = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        if (r < nrows) {
          const size_t at = static_cast<size_t>(pos0 + r) * a.N + n;
          if (a.out_bf16)
            ob[at] = f32_to_bf16(v[r]);
          else
            a.out[at] = v[r];
        }
      }
    }
    return;
  }
  // SwiGLU: columns 0..127 of the tile are gate, 128..255 the matching up columns
  if (mine) {
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      if (r < nrows) tred[r * kGemvCols + t] = v[r];
  }
  __syncthreads();
  const int n = ttile * (kGemvCols / 2) + t;
  if (mine && t < kGemvCols / 2 && n < a.N) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      if (r < nrows) {
        const size_t at = static_cast<size_t>(pos0 + r) * a.N + n;
        const float hv = silu(tred[r * kGemvCols + t]) * tred[r * kGemvCols + kGemvCols / 2 + t];
        if (a.h_bf16)
          reinterpret_cast<uint16_t*>(a.h)[at] = f32_to_bf16(hv);
        else
          a.h[at] = hv;
      }
    }
  }
}

}  // namespace

GemvShape gemv_shape(size_t items, int N, int mode, int G, size_t max_split_tasks) {
  GemvShape sh;
  const int per_tile = mode == 1 ? kGemvCols / 2 : kGemvCols;
  sh.tiles = (N + per_tile - 1) / per_tile;
  const size_t tasks = items * static_cast<size_t>(sh.tiles);
  int S = tasks > 0 ? static_cast<int>(W4_GEMV_TARGET_WGS / tasks) : 1;
  // no more splits than it takes to give each one a full staging window:
  // shorter splits add fixed per-workgroup cost (staging, split-K tail)
  // without adding bandwidth -- unless even one window per split leaves most
  // CUs without a workgroup (one GPU's share of a tensor-parallel MLP at
  // decode size: hidden 7168, intermediate 2304, 29.0 -> 24.8 us per step)
  const int s_window = (G + kWin - 1) / kWin;
  const int s_fill = tasks > 0 ? static_cast<int>((kGemvMinWorkgroups + tasks - 1) / tasks) : 1;
  const int s_cap = tasks * static_cast<size_t>(s_window) < kGemvMinWorkgroups ? s_fill : s_window;
  if (S > s_cap) S = s_cap;
  int max_s = G / W4_GEMV_MIN_GROUPS_PER_SPLIT;
  if (max_s > kMaxSplits) max_s = kMaxSplits;
  if (S > max_s) S = max_s;
  if (tasks > max_split_tasks) S = 1;
  if (S < 1) S = 1;
  sh.gps = G > 0 ? (G + S - 1) / S : 1;
  sh.S = G > 0 ? (G + sh.gps - 1) / sh.gps : 1;  // no empty split
  return sh;
}

int gemv_tiles_per_workgroup(size_t num_tasks, int tiles, int pieces) {
  const int max_kt = pieces == 1 ? 2 : 4;  // the tile buffers of 16-row quads: two fit
  if (W4_GEMV_KT > 0) return W4_GEMV_KT < max_kt ? W4_GEMV_KT : max_kt;
  // A launch that fits one round of four-wave workgroups (four per CU) takes
  // the largest workgroups that still give every CU one; longer launches keep
  // four-wave workgroups, which overlap one's tail with the others' streams.
  if (num_tasks > kGemvResidentTasks || tiles <= 0) return 1;
  const size_t rows_splits = num_tasks / static_cast<size_t>(tiles);
  for (int kt = max_kt; kt > 1; kt /= 2)
    if (rows_splits * ((tiles + kt - 1) / kt) >= kGemvMinWorkgroups) return kt;
  return 1;
}

namespace {
void launch_kt(const GemvArgs& a, int kt, unsigned blocks, hipStream_t stream, hipEvent_t start,
               hipEvent_t stop) {
  if (a.pieces == 1) {
    if (kt == 2)
      hipExtLaunchKernelGGL(gemv_kernel<2, 1>, dim3(blocks), dim3(kGemvThreads * 2), 0, stream, start, stop, 0,
                            a);
    else
      hipExtLaunchKernelGGL(gemv_kernel<1, 1>, dim3(blocks), dim3(kGemvThreads), 0, stream, start, stop, 0, a);
    return;
  }
  switch (kt) {
    case 4:
      hipExtLaunchKernelGGL(gemv_kernel<4, 2>, dim3(blocks), dim3(kGemvThreads * 4), 0, stream, start, stop, 0,
                            a);
      break;
    case 2:
      hipExtLaunchKernelGGL(gemv_kernel<2, 2>, dim3(blocks), dim3(kGemvThreads * 2), 0, stream, start, stop, 0,
                            a);
      break;
    default:
      hipExtLaunchKernelGGL(gemv_kernel<1, 2>, dim3(blocks), dim3(kGemvThreads), 0, stream, start, stop, 0, a);
      break;
  }
}
}  // namespace

w4a16_status_t launch_gemv(const GemvArgs& a, size_t num_tasks, hipStream_t stream, hipEvent_t start,
                           hipEvent_t stop) {
  if (num_tasks == 0) return W4A16_OK;
  if (a.tiles <= 0 || a.S <= 0 || num_tasks % (static_cast<size_t>(a.tiles) * a.S) != 0)
    return W4A16_ERR_INVALID_ARG;
  if (a.pieces != 1 && a.pieces != 2) return W4A16_ERR_INVALID_ARG;
  const int kt = gemv_tiles_per_workgroup(num_tasks, a.tiles, a.pieces);
  const size_t blocks = num_tasks / a.tiles * ((a.tiles + kt - 1) / kt);
  if (blocks > 0x7fffffffu) return W4A16_ERR_UNSUPPORTED;
  launch_kt(a, kt, static_cast<unsigned>(blocks), stream, start, stop);
  return launch_status();
}

}  // namespace w4
