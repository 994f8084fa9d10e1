// Split-K GEMV for decode-sized row counts (internal interface).
#pragma once

#include "common.h"

namespace w4 {

// Activation rows enter the GEMV as signed fixed point per (row, 32-row group):
// X = rint(x * 2^sh) with |X| <= 2^(8P-2), split into P signed bytes
// (X = sum_p piece_p * 256^(P-1-p)).  P = 3 keeps float32 activations to
// 2^-23 of the group's largest magnitude, P = 2 keeps bf16 activations to
// 2^-15.  Per (row, group) the pieces take 8P dwords laid out as
// [piece][word j][parity], byte b of dword (p, j, par) holding element
// k = 8j + 2b + par; the float factor 2^-(sh+4) undoes the scaling and the
// x16 carried by the byte-expanded weights.
//
// Pieces are stored group-major by position: xq[g][pos][8P], xf[g][pos], so
// the rows of one task are adjacent and one scalar base pointer with
// immediate offsets reaches all of them.  Positions are token rows for a
// dense call and (expert, token) pairs in routed order for the MoE.
inline int pieces_for(w4a16_dtype_t xt) { return xt == W4A16_F32 ? 3 : 2; }

struct GemvArgs {
  const int32_t* xq;   // [G][R][8P] pieces of the input positions
  const float* xf;     // [G][R] factors
  int G;               // groups along K (K / 32)
  int R;               // positions held in xq / xf
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
  int32_t* hq;           // SwiGLU: pieces of h, [N/32][R][8P]
  float* hf;             // SwiGLU: factors of h, [N/32][R]
  void* h_raw;           // SwiGLU, optional: h[position][N] as float32 or bf16
  int h_bf16;
  float* partials;       // split-K partial tiles
  int* counters;         // split-K arrival counters (zero between calls)
};

constexpr int kGemvThreads = 256;
constexpr size_t kPartialTileFloats = static_cast<size_t>(kMaxGemvRows) * 64;

// Pieces of R positions.  With sorted_pairs == nullptr position p is row p of
// x; otherwise it is row sorted_pairs[p] / top_k, and a negative pair id gives
// zero pieces and a zero factor.
w4a16_status_t launch_prep_pieces(const void* x, w4a16_dtype_t xt, int R, int K, int P,
                                  const int* sorted_pairs, int top_k, int32_t* xq, float* xf,
                                  hipStream_t stream);
w4a16_status_t launch_gemv(const GemvArgs& a, int P, size_t num_tasks, hipStream_t stream);

// Split count for a GEMV over `tasks` (item, tile) pairs with G groups.
int gemv_splits(size_t tasks, int G);

}  // namespace w4
