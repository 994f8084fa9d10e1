// MFMA tile GEMM for row counts above the GEMV range (internal interface).
#pragma once

#include "common.h"

namespace w4 {

// Activations enter the MFMA kernel as f16 "pieces" of a per-row power-of-two
// rescaling: v = x * 2^e with max|x_row| * 2^e in [2^14, 2^15), piece 0 =
// f16(v), piece 1 = f16(v - piece 0) (float32 activations only).  Two pieces
// carry 22 significant bits; bf16 activations fit in one.  Within every block
// of 8 consecutive k the pieces are stored in the order k = 0,4,1,5,2,6,3,7,
// the order in which one packed code word expands into f16 pairs.
// Layout: ap[p][Mp][K] f16, rs[Mp] = 2^-e (0 for an all-zero or absent row).
inline int mfma_pieces(w4a16_dtype_t xt) { return xt == W4A16_F32 ? 2 : 1; }

constexpr int kMfmaRows = 64;     // rows per tile
constexpr int kMfmaCols = 256;    // weight columns per tile (4 waves x 4 blocks of 16)
constexpr int kMfmaThreads = 256;
// Workgroups of the tile kernel resident at once (two per CU on 256 CUs) and
// the fixed cost of one workgroup (staging, the store of its 64 KiB of split
// sums and their later read, epilogue) in units of one group step (about 5 KiB
// of weights); the split planner balances launches with them.
#ifndef W4_MFMA_WG_OVERHEAD_GROUPS
#define W4_MFMA_WG_OVERHEAD_GROUPS 16
#endif
#ifndef W4_MFMA_PARTIAL_CAP
#define W4_MFMA_PARTIAL_CAP 1.0  // split-sum traffic cap, a fraction of the weight bytes
#endif
constexpr int kMfmaResidentWgs = 512;

// Wide tiles (wide.hip): 256 rows x 128 columns per workgroup, bf16
// activations, dense rows, plain output; taken from W4_WIDE_MIN_ROWS rows on.
constexpr int kWideRows = 256;
constexpr int kWideCols = 128;
constexpr int kWideThreads = 256;
#ifndef W4_WIDE_MIN_ROWS
#define W4_WIDE_MIN_ROWS 256
#endif
constexpr int kWideResidentWgs = 256;  // one per CU
constexpr int kMfmaWgOverheadGroups = W4_MFMA_WG_OVERHEAD_GROUPS;

struct MfmaArgs {
  const _Float16* ap;  // [P][Mp][K]
  const float* rs;     // [Mp]
  int Mp;              // rows per piece plane (a multiple of 64, >= positions + 64, or the token count)
  // Optional: position p takes piece row arow[min(p, arow_n - 1)] / arow_div
  // (the token of a routed pair) instead of row p.
  const int* arow;
  int arow_div, arow_n;
  int K, G;
  const u32x4* qw0;    // GROUPED chunks, matrix 0 (plain, or gate)
  const float* sc0;
  const u32x4* qw1;    // up (SwiGLU mode)
  const float* sc1;
  size_t expert_stride;  // chunks per expert (scales per expert: expert_stride >> gshift)
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
  int S, gps;            // K splits, groups per split
  int dense_rows;        // > 0: dense rows, items of 64 rows
  const int4* items;     // grouped mode: {expert, first position, rows, 0}
  const int* n_items;
  int mode;              // 0: plain out[pos][N]; 1: SwiGLU, h[pos][N]
  float* out;            // float32, or bf16 (round to nearest even) with out_bf16
  int out_bf16;
  float* h;              // SwiGLU output h[pos][N]: float32, or bf16 with h_bf16
  int h_bf16;
  float* partials;
  int* counters;
  // Deferred split-K (dense launches with S > 1): with `planes` set, each
  // workgroup stores its sums to planes[split][m][row][plane_ld] (m: 0 plain
  // or gate, 1 up; rows of the item plane) and the reduction runs in the
  // next kernel (launch_plane_sum, or the h pieces of launch_prep_planes).
  float* planes;
  int plane_rows, plane_ld;
};

// Pieces of R positions (rows of x, or gathered rows gather[p] / top_k); rows
// R .. Mp-1 are zero-filled.  With `need` set, only positions p < R with
// need[p] != 0 are written (the others are never read).
w4a16_status_t launch_mfma_prep(const void* x, w4a16_dtype_t xt, int R, int Mp, int K, int P,
                                const int* gather, int top_k, const int* need, _Float16* ap,
                                float* rs, hipStream_t stream, hipEvent_t start = nullptr,
                                hipEvent_t stop = nullptr);
// start / stop (optional) are recorded at the kernel's own start and end.
w4a16_status_t launch_mfma(const MfmaArgs& a, int P, size_t num_tasks, hipStream_t stream,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Wide-tile launch (mode 0, dense rows, Mp a multiple of kWideRows); a.tiles
// counts 128-column tiles.
w4a16_status_t launch_wide(const MfmaArgs& a, size_t num_tasks, hipStream_t stream, hipEvent_t start = nullptr,
                           hipEvent_t stop = nullptr);

// Deferred split-K, plain output: out[m][n] = (sum over splits, in split
// order, of planes[s][0][m][n]) * rs[m] for m < M, n < N (N a multiple of 4);
// with rs_stride > 0, the split-order sum of planes[s][0][m][n] *
// rs[s * rs_stride + m] (activations scaled per row and split).
w4a16_status_t launch_plane_sum(const float* planes, int S, int plane_rows, int plane_ld, const float* rs,
                                int rs_stride, int M, int N, float* out, hipStream_t stream,
                                hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Deferred split-K, SwiGLU: h[m][n] = silu(g * f) * (u * f) with g, u the
// split-order sums of planes[s][0] and planes[s][1] and f = rsx[m], written
// to h[M][I], then the f16 pieces of h as launch_mfma_prep makes them
// (rows M .. Mp-1 zero-filled).
w4a16_status_t launch_prep_planes(const float* planes, int S, int plane_rows, int plane_ld, const float* rsx,
                                  int M, int Mp, int I, int P, float* h, _Float16* ap, float* rs,
                                  hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Deferred split-K, SwiGLU, pieces per down split: the h columns [c * cols,
// (c + 1) * cols) of row m, h = silu(g * f) * (u * f) as above, become f16
// pieces scaled to that range's own largest magnitude, rs[c * Mp + m] =
// 2^-e (rows M .. Mp-1: zero pieces, rs 0).  h itself is not stored.
// UNSUPPORTED when a range holds more than split_pieces_threads' limit
// (256 threads x 4 blocks of 8 = 8192 columns).
int split_pieces_threads(int cols);  // 0: range too long
w4a16_status_t launch_prep_split_pieces(const float* planes, int S, int plane_rows, int plane_ld, const float* rsx,
                                        int M, int Mp, int I, int P, int cols, _Float16* ap, float* rs,
                                        hipStream_t stream, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);

// Rows of the piece planes for R positions.
inline int mfma_rows_padded(int R) { return (R + kMfmaRows - 1) / kMfmaRows * kMfmaRows + kMfmaRows; }

}  // namespace w4
