// Split-K GEMV for decode-sized row counts (internal interface).
#pragma once

#include "common.h"

namespace w4 {

// Activations enter the GEMV as signed fixed point per (row, 32-row group):
// X = rint(x * 2^sh), split into D balanced signed 4-bit digits,
// X = sum_d digit_d * 16^(D-1-d), digit in [-8, 7].  sh is the largest integer
// with max|x| * 2^sh <= 3 * 2^(4D-3), which keeps every digit in range and the
// rounding error below 2^-(4D-2) of the group's largest magnitude.  D = 5 for
// float32 activations (20 bits), D = 4 for bf16 (16 bits, above bf16's 8).
// Per (row, group) the digits take 4D dwords, dword (d, j) holding digit d of
// elements k = 8j .. 8j+7 in nibble order, plus one float factor 2^-sh.
//
// Digits made by one kernel for another (the SwiGLU epilogue's output) are
// stored group-major by position: xq[g][pos][4D], xf[g][pos], so the rows of
// one task are adjacent.
inline int digits_for(w4a16_dtype_t xt) { return xt == W4A16_F32 ? 5 : 4; }

enum GemvInput : int {
  kInDigits = 0,  // xq / xf digits (group-major by position)
  kInF32 = 1,     // float32 rows of x, optionally gathered
  kInBF16 = 2,    // bf16 rows of x, optionally gathered
};

struct GemvArgs {
  const void* x;       // raw activations [rows][K] (kInF32 / kInBF16)
  const int* gather;   // raw input: position p reads row gather[p] / top_k (nullptr: row p)
  int top_k;
  const int32_t* xq;   // kInDigits: [G][R][4D]
  const float* xf;     // kInDigits: [G][R]
  int G;               // groups along K (K / 32)
  int K;
  int R;               // positions held in xq / xf and produced into hq / hf
  const u32x4* qw0;    // GROUPED chunks, matrix 0 (plain, or gate)
  const float* sc0;
  const u32x4* qw1;    // matrix 1 (up) for the SwiGLU mode, else null
  const float* sc1;
  size_t expert_stride;  // chunks (and scales) per expert: G * N
  int N;                 // columns per matrix
  int tiles;             // column tiles per row item
  int S;                 // K splits across workgroups
  int gps;               // groups per split
  int dense_rows;        // > 0: dense rows 0..dense_rows-1, items of 8 rows
  const int4* items;     // grouped mode: {expert, first position, rows, 0}
  const int* n_items;    // grouped mode: number of valid items (device)
  int mode;              // 0: plain float32 output, 1: SwiGLU epilogue
  float* out;            // plain: out[position][N]
  int32_t* hq;           // SwiGLU: digits of h, [N/32][R][4D]
  float* hf;             // SwiGLU: factors of h, [N/32][R]
  void* h_raw;           // SwiGLU, optional: h[position][N] as float32 or bf16
  int h_bf16;
  float* partials;       // split-K partial tiles
  int* counters;         // split-K arrival counters (zero between calls)
};

constexpr int kGemvThreads = 256;
constexpr int kMaxSplits = 32;  // K splits of one GEMV (partials read back together)

// Launch-shape defaults (overridable at compile time for tuning sweeps).
#ifndef W4_GEMV_TARGET_WGS
#define W4_GEMV_TARGET_WGS 1024
#endif
#ifndef W4_GEMV_MIN_GROUPS_PER_WAVE
#define W4_GEMV_MIN_GROUPS_PER_WAVE 6
#endif
#ifndef W4_GEMV_SUB
#define W4_GEMV_SUB 4
#endif
#ifndef W4_GEMV_WAVES_PER_EU
#define W4_GEMV_WAVES_PER_EU 4
#endif

// Launch shape of one GEMV: columns per lane, column tiles per row item, K
// splits.  Chosen so the grid fills the resident capacity of the GPU (about
// W4_GEMV_TARGET_WGS workgroups) as evenly as possible, preferring more
// columns per lane (fewer LDS reads per dot product) when the fill is similar.
struct GemvShape {
  int sub = 1, tiles = 1, S = 1;
};
GemvShape gemv_shape(size_t items, int N, int mode, int G, size_t max_split_tasks);

// floats of one split-K partial tile
inline size_t partial_tile_floats(int sub) { return static_cast<size_t>(kMaxGemvRows) * 64 * sub; }

w4a16_status_t launch_gemv(const GemvArgs& a, int D, int SUB, int input, size_t num_tasks,
                           hipStream_t stream);


}  // namespace w4
