// Split-K MFMA GEMV for decode-sized row counts (internal interface).
#pragma once

#include "common.h"

namespace w4 {

// One task covers up to gemv_rows(pieces) positions (rows) of one item, one column
// tile and one K split.  Activations are read raw (float32 or bf16) and turned
// into f16 pieces inside the kernel, one staging window of groups at a time.
struct GemvArgs {
  const void* x;        // activations [rows][K], float32 or bf16
  int x_bf16;
  int pieces;           // f16 pieces per activation: 2 (tasks of 8 rows) or 1 (tasks of 16 rows)
  const int* gather;    // position p reads row gather[p] / top_k (negative: a zero row);
  int top_k;            //   nullptr: position p reads row p
  int K, G;             // G = K / 32
  const u32x4* qw0;     // GROUPED chunks, matrix 0 (plain, or gate)
  const float* sc0;
  const u32x4* qw1;     // matrix 1 (up) for the SwiGLU mode, else null
  const float* sc1;
  size_t expert_stride;  // chunks per expert: G * N (scales per expert: expert_stride >> gshift)
  int gshift;            // scale group = 32 << gshift rows: scale row of code block g is g >> gshift
  // One more expert with weights of its own (the shared expert of an MoE
  // layer): id extra_plus1 - 1 reads these instead of the stacks (0: none).
  int extra_plus1;
  const u32x4* qw0x;
  const float* sc0x;
  const u32x4* qw1x;
  const float* sc1x;
  int N;                 // columns per matrix
  int tiles;             // column tiles per row item
  int S;                 // K splits across workgroups
  int gps;               // groups per split
  int dense_rows;        // > 0: dense rows 0..dense_rows-1, items of gemv_rows(pieces) rows
  const int4* items;     // grouped mode: {expert, first position, rows, 0}
  const int* n_items;    // grouped mode: number of valid items (device)
  int mode;              // 0: plain, out[position][N]; 1: SwiGLU, h[position][N]
  float* out;            // float32, or bf16 (round to nearest even) with out_bf16
  int out_bf16;
  float* h;              // SwiGLU output h = silu(x Wg) * (x Wu): float32, or bf16 with h_bf16
  int h_bf16;
  float* partials;       // split-K partial tiles
  int* counters;         // split-K arrival counters (zero between calls)
};

constexpr int kGemvThreads = 256;
constexpr int kGemvCols = 256;     // weight columns per tile (4 waves x 64)
constexpr int kMaxSplits = 32;

// Launch-shape defaults (overridable at compile time for tuning sweeps).
#ifndef W4_GEMV_TARGET_WGS
#define W4_GEMV_TARGET_WGS 1024
#endif
#ifndef W4_GEMV_MIN_GROUPS_PER_SPLIT
#define W4_GEMV_MIN_GROUPS_PER_SPLIT 8
#endif

// Launch shape of one GEMV: column tiles per row item and K splits, chosen so
// the grid fills about W4_GEMV_TARGET_WGS resident workgroups.
struct GemvShape {
  int tiles = 1, S = 1, gps = 1;
};
GemvShape gemv_shape(size_t items, int N, int mode, int G, size_t max_split_tasks);

// floats of one split-K partial tile (room for 16 rows)
constexpr size_t kPartialTileFloats = static_cast<size_t>(kGemvRowsOnePiece) * kGemvCols;

// Pieces per activation and rows per task of the GEMV for an activation type:
// bf16 fits one f16 piece exactly (16 rows per task), float32 takes two (8).
inline int gemv_pieces(w4a16_dtype_t xt) { return xt == W4A16_BF16 ? 1 : 2; }
inline int gemv_rows(w4a16_dtype_t xt) { return xt == W4A16_BF16 ? kGemvRowsOnePiece : kMaxGemvRows; }

#ifndef W4_GEMV_KT
#define W4_GEMV_KT 0  // column tiles per workgroup; 0: chosen per launch
#endif
constexpr size_t kGemvResidentTasks = 1024;  // four-wave workgroups resident at once (4 per CU)
constexpr size_t kGemvMinWorkgroups = 240;   // about one workgroup per CU

// Column tiles per workgroup (1, 2 or 4 quads of four waves; at most 2 with
// one piece) for a launch of num_tasks = items * tiles * S tasks.
int gemv_tiles_per_workgroup(size_t num_tasks, int tiles, int pieces);
// num_tasks must be items * a.tiles * a.S.
// start / stop (optional) are recorded at the kernel's own start and end.
w4a16_status_t launch_gemv(const GemvArgs& a, size_t num_tasks, hipStream_t stream,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

}  // namespace w4
