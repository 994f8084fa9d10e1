// Host entry points: argument checks, workspace layout and kernel dispatch for
// the dense GEMM and the dense SwiGLU MLP.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "dispatch.h"

namespace w4 {

// ---------------------------------------------------------------- workspace layout

void Carve::take(size_t& off, size_t bytes) {
  off = cursor;
  cursor = round_up(cursor + bytes, 256);
}

size_t gemv_partial_bytes(size_t tasks, int S) {
  return S > 1 ? tasks * S * kPartialTileFloats * sizeof(float) : 0;
}

MfmaPlan plan_wide(int rows, int N, int K) {
  MfmaPlan m;
  m.wide = true;
  m.P = 1;
  m.Mp = static_cast<int>(round_up(static_cast<size_t>(rows), kWideRows));
  m.items = static_cast<size_t>(m.Mp / kWideRows);
  m.tiles = (N + kWideCols - 1) / kWideCols;
  m.tasks = m.items * m.tiles;
  const int G = K / kGroup;
  // split K until the grid holds about one workgroup per CU, keeping at least
  // 16 groups per split
  int S = 1;
  while (m.tasks * (S + 1) <= static_cast<size_t>(kWideResidentWgs) && (S + 1) * 16 <= G && S + 1 <= kMaxSplits &&
         m.tasks * (S + 1) * sizeof(int) <= kCounterBytes)
    ++S;
  if (m.tasks * sizeof(int) > kCounterBytes) S = 1;
  // a multiple of four groups per split (G is one): whole four-group windows
  m.gps = G > 0 ? ((G + S - 1) / S + 3) / 4 * 4 : 4;
  m.S = G > 0 ? (G + m.gps - 1) / m.gps : 1;
  return m;
}

MfmaPlan plan_mfma(int rows, int N, int mode, int K, w4a16_dtype_t xt, bool allow_wide) {
  // (the wide kernel's buffer offsets are 32-bit: codes under 2 GiB)
  if (allow_wide && xt == W4A16_BF16 && mode == 0 && rows >= W4_WIDE_MIN_ROWS && K % 128 == 0 &&
      static_cast<size_t>(K) * N / 2 < (size_t{1} << 31))
    return plan_wide(rows, N, K);
  MfmaPlan m;
  m.P = mfma_pieces(xt);
  m.Mp = mfma_rows_padded(rows);
  m.items = (static_cast<size_t>(rows) + kMfmaRows - 1) / kMfmaRows;
  const int per_tile = mode == 1 ? kMfmaCols / 2 : kMfmaCols;
  m.tiles = (N + per_tile - 1) / per_tile;
  m.tasks = m.items * m.tiles;
  const int G = K / kGroup;
  // Split K to balance the grid over the resident workgroups: the kernel holds
  // two workgroups per CU (its registers allow two waves per SIMD), 512 on
  // the chip, and every workgroup of a launch streams the same number of
  // groups, so a launch takes about ceil(tasks * S / 512) rounds of
  // (G / S + a fixed per-workgroup cost) group steps.  The split sums' write
  // + read traffic stays under the weight bytes.
  const double wbytes_per_col = K * 0.625;
  const double part_per_col_per_split = 8.0 * static_cast<double>(m.items) * kMfmaRows;
  int s_max = static_cast<int>(W4_MFMA_PARTIAL_CAP * wbytes_per_col / part_per_col_per_split);
  // A grid that would leave more than half the CUs idle may split past the
  // cap (one GPU's share of a tensor-parallel MLP at M = 64: its down
  // projection has 28 column tiles and a cap of 2 splits; 51.7 -> 48.2 us).
  const int s_fill = static_cast<int>((kMfmaResidentWgs / 4 + m.tasks - 1) / m.tasks);
  if (s_max < s_fill) s_max = s_fill;
  if (s_max > G / 4) s_max = G / 4;
  if (s_max > kMaxSplits) s_max = kMaxSplits;
  while (s_max > 1 && m.tasks * s_max * sizeof(int) > kCounterBytes) --s_max;
  int S = 1;
  double best = 0.0;
  for (int s = 1; s <= std::max(s_max, 1); ++s) {
    const double rounds = std::ceil(static_cast<double>(m.tasks) * s / kMfmaResidentWgs);
    const double cost = rounds * ((G + s - 1) / s + kMfmaWgOverheadGroups);
    if (s == 1 || cost < best) {
      best = cost;
      S = s;
    }
  }
  // the tile kernel addresses a split's codes with 32-bit buffer offsets
  const size_t row_bytes = static_cast<size_t>(N) * 16;
  while (S < G && static_cast<size_t>((G + S - 1) / S) * row_bytes > 0x7fffffffu) ++S;
  m.S = S;
  m.gps = (G + S - 1) / S;
  return m;
}

size_t mfma_partial_bytes(const MfmaPlan& m) {
  if (m.wide) return m.S > 1 ? m.tasks * m.S * static_cast<size_t>(kWideRows) * kWideCols * sizeof(float) : 0;
  return m.S > 1 ? m.tasks * m.S * static_cast<size_t>(kMfmaRows) * kMfmaCols * sizeof(float) : 0;
}

MfmaArgs mfma_dense_args(const MfmaPlan& m, int rows, const w4a16_weight_t* w0,
                         const w4a16_weight_t* w1, int mode, const _Float16* ap, const float* rs,
                         char* ws, size_t partials_off, size_t counters_off) {
  MfmaArgs a{};
  a.ap = ap;
  a.rs = rs;
  a.Mp = m.Mp;
  a.K = w0->K;
  a.G = w0->K / kGroup;
  a.qw0 = reinterpret_cast<const u32x4*>(w0->qw);
  a.sc0 = w0->scales;
  if (w1 != nullptr) {
    a.qw1 = reinterpret_cast<const u32x4*>(w1->qw);
    a.sc1 = w1->scales;
  }
  a.N = w0->N;
  a.tiles = m.tiles;
  a.S = m.S;
  a.gps = m.gps;
  a.gshift = group_shift(w0);
  a.dense_rows = rows;
  a.mode = mode;
  a.partials = reinterpret_cast<float*>(ws + partials_off);
  a.counters = reinterpret_cast<int*>(ws + counters_off);
  return a;
}

// Deferred split-K for a dense tile launch with S > 1: the split sums go to
// planes in the partials region (the same bytes as the partial tiles) and the
// next kernel reduces them in split order.
void defer_split_k(MfmaArgs& a, const MfmaPlan& m) {
  a.planes = a.partials;
  a.plane_rows = static_cast<int>(m.items) * kMfmaRows;
  a.plane_ld = m.tiles * (a.mode == 1 ? kMfmaCols / 2 : kMfmaCols);
}

GemmPlan plan_gemm(int M, const w4a16_weight_t* w, w4a16_dtype_t xt) {
  GemmPlan p;
  if (M > gemv_rows(xt)) {
    p.mfma = true;
    p.mf = plan_mfma(M, w->N, 0, w->K, xt, true);
    Carve c;
    c.take(p.counters_off, kCounterBytes);
    // (wide tiles read up to 128 bytes past the piece plane: padded)
    c.take(p.ap_off, static_cast<size_t>(p.mf.P) * p.mf.Mp * w->K * 2 + (p.mf.wide ? 256 : 0));
    c.take(p.rs_off, static_cast<size_t>(p.mf.Mp) * 4);
    c.take(p.partials_off, mfma_partial_bytes(p.mf));
    p.bytes = c.cursor;
    return p;
  }
  const int G = w->K / kGroup;
  const size_t items = (static_cast<size_t>(M) + gemv_rows(xt) - 1) / gemv_rows(xt);
  const GemvShape sh = gemv_shape(items, w->N, 0, G, kCounterBytes / sizeof(int));
  p.tiles = sh.tiles;
  p.tasks = items * p.tiles;
  p.S = sh.S;
  p.gps = sh.gps;
  Carve c;
  c.take(p.counters_off, kCounterBytes);
  c.take(p.partials_off, gemv_partial_bytes(p.tasks, p.S));
  p.bytes = c.cursor;
  return p;
}

MlpPlan plan_mlp(int M, w4a16_dtype_t xt, const w4a16_weight_t* gate, const w4a16_weight_t* down) {
  MlpPlan p;
  if (M > gemv_rows(xt)) {
    const int H = gate->K, I = gate->N;
    p.mfma = true;
    p.gu = plan_mfma(M, I, 1, H, xt, false);
    p.dn = plan_mfma(M, down->N, 0, I, xt, false);
    const int P = p.gu.P, Mp = p.gu.Mp;
    // Both launches split K: h's pieces are made per down split, from the
    // gate/up split sums, and h itself is never stored.
    p.split_pieces = p.gu.S > 1 && p.dn.S > 1 && split_pieces_threads(p.dn.gps * kGroup) > 0;
    Carve c;
    c.take(p.counters_off, kCounterBytes);
    c.take(p.apx_off, static_cast<size_t>(P) * Mp * H * 2);
    c.take(p.rsx_off, static_cast<size_t>(Mp) * 4);
    c.take(p.h_off, p.split_pieces ? 0 : static_cast<size_t>(Mp) * I * 4);
    c.take(p.aph_off, static_cast<size_t>(P) * Mp * I * 2);
    c.take(p.rsh_off, static_cast<size_t>(Mp) * (p.split_pieces ? p.dn.S : 1) * 4);
    c.take(p.partials_off, std::max(mfma_partial_bytes(p.gu), mfma_partial_bytes(p.dn)));
    p.bytes = c.cursor;
    return p;
  }
  const int H = gate->K, I = gate->N;
  const int GH = H / kGroup, GI = I / kGroup;
  const size_t items = (static_cast<size_t>(M) + gemv_rows(xt) - 1) / gemv_rows(xt);
  const GemvShape gu = gemv_shape(items, I, 1, GH, kCounterBytes / sizeof(int));
  p.tiles_gu = gu.tiles;
  p.tasks_gu = items * p.tiles_gu;
  p.S_gu = gu.S;
  p.gps_gu = gu.gps;
  const GemvShape dn = gemv_shape(items, down->N, 0, GI, kCounterBytes / sizeof(int));
  p.tiles_d = dn.tiles;
  p.tasks_d = items * p.tiles_d;
  p.S_d = dn.S;
  p.gps_d = dn.gps;
  Carve c;
  c.take(p.counters_off, kCounterBytes);
  c.take(p.h_off, static_cast<size_t>(M) * I * 4);
  c.take(p.partials_off, std::max(gemv_partial_bytes(p.tasks_gu, p.S_gu), gemv_partial_bytes(p.tasks_d, p.S_d)));
  p.bytes = c.cursor;
  return p;
}

bool counters_fit(size_t tasks, int S) {
  return S <= 1 || tasks * sizeof(int) <= kCounterBytes;
}

w4a16_status_t check_dense_grouped(const w4a16_weight_t* w) {
  w4a16_status_t st = check_weight(w);
  if (st != W4A16_OK) return st;
  if (w->layout != W4A16_LAYOUT_GROUPED || w->num_experts != 1) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

bool ranges_overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return abytes && bbytes && a0 < b0 + bbytes && b0 < a0 + abytes;
}

size_t dtype_bytes(w4a16_dtype_t xt) { return xt == W4A16_F32 ? 4 : 2; }

GemvArgs gemv_dense_args(int M, const w4a16_weight_t* w0, const w4a16_weight_t* w1, int mode,
                         const void* x, bool x_bf16, int pieces, int tiles, int S, int gps, char* ws,
                         size_t partials_off, size_t counters_off) {
  GemvArgs a{};
  a.x = x;
  a.x_bf16 = x_bf16 ? 1 : 0;
  a.pieces = pieces;
  a.G = w0->K / kGroup;
  a.K = w0->K;
  a.qw0 = reinterpret_cast<const u32x4*>(w0->qw);
  a.sc0 = w0->scales;
  if (w1 != nullptr) {
    a.qw1 = reinterpret_cast<const u32x4*>(w1->qw);
    a.sc1 = w1->scales;
  }
  a.expert_stride = 0;
  a.N = w0->N;
  a.tiles = tiles;
  a.S = S;
  a.gps = gps;
  a.gshift = group_shift(w0);
  a.dense_rows = M;
  a.mode = mode;
  a.partials = reinterpret_cast<float*>(ws + partials_off);
  a.counters = reinterpret_cast<int*>(ws + counters_off);
  return a;
}

}  // namespace w4

using namespace w4;

extern "C" size_t w4a16_gemm_workspace_bytes(int32_t M, const w4a16_weight_t* w, w4a16_dtype_t xt) {
  if (M <= 0 || check_dense_grouped(w) != W4A16_OK) return 0;
  if (xt != W4A16_F32 && xt != W4A16_BF16) return 0;
  return plan_gemm(M, w, xt).bytes;
}

namespace w4 {
static w4a16_status_t gemm_impl(const void* x, w4a16_dtype_t xt, int32_t M, const w4a16_weight_t* w, float* y,
                                void* ws, size_t ws_bytes, hipStream_t stream, EventMarks& ev) {
  w4a16_status_t st = check_dense_grouped(w);
  if (st != W4A16_OK) return st;
  if (M < 0 || (xt != W4A16_F32 && xt != W4A16_BF16)) return W4A16_ERR_INVALID_ARG;
  if (M == 0 || w->K == 0 || w->N == 0) return W4A16_OK;
  if (x == nullptr || y == nullptr || ws == nullptr) return W4A16_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return W4A16_ERR_INVALID_ARG;
  if (ranges_overlap(x, static_cast<size_t>(M) * w->K * dtype_bytes(xt), y,
                     static_cast<size_t>(M) * w->N * 4))
    return W4A16_ERR_INVALID_ARG;
  const GemmPlan p = plan_gemm(M, w, xt);
  if (ws_bytes < p.bytes) return W4A16_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(ws);
  if (p.mfma) {
    _Float16* ap = reinterpret_cast<_Float16*>(wsb + p.ap_off);
    float* rs = reinterpret_cast<float*>(wsb + p.rs_off);
    EventMarks::Bracket b = ev.bracket();
    st = launch_mfma_prep(x, xt, M, p.mf.Mp, w->K, p.mf.P, nullptr, 0, nullptr, ap, rs, stream, b.start, b.stop);
    if (st != W4A16_OK) return st;
    MfmaArgs a = mfma_dense_args(p.mf, M, w, nullptr, 0, ap, rs, wsb, p.partials_off, p.counters_off);
    a.out = y;
    b = ev.bracket();
    if (p.mf.wide) return launch_wide(a, p.mf.tasks * p.mf.S, stream, b.start, b.stop);
    if (p.mf.S == 1) return launch_mfma(a, p.mf.P, p.mf.tasks * p.mf.S, stream, b.start, b.stop);
    defer_split_k(a, p.mf);
    st = launch_mfma(a, p.mf.P, p.mf.tasks * p.mf.S, stream, b.start, b.stop);
    if (st != W4A16_OK) return st;
    b = ev.bracket();
    return launch_plane_sum(a.planes, a.S, a.plane_rows, a.plane_ld, rs, 0, M, w->N, y, stream, b.start, b.stop);
  }
  if (!counters_fit(p.tasks, p.S)) return W4A16_ERR_UNSUPPORTED;
  GemvArgs a = gemv_dense_args(M, w, nullptr, 0, x, xt == W4A16_BF16, gemv_pieces(xt), p.tiles, p.S, p.gps, wsb,
                               p.partials_off, p.counters_off);
  a.out = y;
  EventMarks::Bracket b = ev.bracket();
  return launch_gemv(a, p.tasks * p.S, stream, b.start, b.stop);
}
}  // namespace w4

extern "C" w4a16_status_t w4a16_gemm(const void* x, w4a16_dtype_t xt, int32_t M,
                                     const w4a16_weight_t* w, float* y, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  EventMarks none;
  return gemm_impl(x, xt, M, w, y, ws, ws_bytes, stream, none);
}

extern "C" w4a16_status_t w4a16_gemm_timed(const void* x, w4a16_dtype_t xt, int32_t M,
                                           const w4a16_weight_t* w, float* y, void* ws, size_t ws_bytes,
                                           hipStream_t stream, hipEvent_t* events, int32_t capacity,
                                           int32_t* recorded) {
  if (capacity < 0 || (capacity > 0 && events == nullptr)) return W4A16_ERR_INVALID_ARG;
  EventMarks ev;
  ev.events = events;
  ev.capacity = capacity;
  const w4a16_status_t st = gemm_impl(x, xt, M, w, y, ws, ws_bytes, stream, ev);
  if (recorded != nullptr) *recorded = ev.recorded;
  return st;
}

extern "C" size_t w4a16_swiglu_mlp_workspace_bytes(int32_t M, w4a16_dtype_t xt,
                                                   const w4a16_weight_t* gate,
                                                   const w4a16_weight_t* up,
                                                   const w4a16_weight_t* down) {
  if (M <= 0 || check_mlp(gate, up, down) != W4A16_OK) return 0;
  if (xt != W4A16_F32 && xt != W4A16_BF16) return 0;
  return plan_mlp(M, xt, gate, down).bytes;
}

namespace w4 {
w4a16_status_t check_mlp(const w4a16_weight_t* gate, const w4a16_weight_t* up,
                         const w4a16_weight_t* down) {
  w4a16_status_t st;
  if ((st = check_dense_grouped(gate)) != W4A16_OK) return st;
  if ((st = check_dense_grouped(up)) != W4A16_OK) return st;
  if ((st = check_dense_grouped(down)) != W4A16_OK) return st;
  if (gate->K != up->K || gate->N != up->N) return W4A16_ERR_UNSUPPORTED;
  if (gate->group_size != up->group_size) return W4A16_ERR_UNSUPPORTED;  // one launch streams both
  if (down->K != gate->N || down->N != gate->K) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}
}  // namespace w4

namespace w4 {
static w4a16_status_t swiglu_mlp_impl(const void* x, w4a16_dtype_t xt, int32_t M,
                                      const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                      const w4a16_weight_t* down, float* y, void* ws,
                                      size_t ws_bytes, hipStream_t stream, EventMarks& ev) {
  w4a16_status_t st = check_mlp(gate, up, down);
  if (st != W4A16_OK) return st;
  if (M < 0 || (xt != W4A16_F32 && xt != W4A16_BF16)) return W4A16_ERR_INVALID_ARG;
  if (M == 0 || gate->K == 0 || gate->N == 0) return W4A16_OK;
  if (x == nullptr || y == nullptr || ws == nullptr) return W4A16_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(ws)) return W4A16_ERR_INVALID_ARG;
  if (ranges_overlap(x, static_cast<size_t>(M) * gate->K * dtype_bytes(xt), y,
                     static_cast<size_t>(M) * gate->K * 4))
    return W4A16_ERR_INVALID_ARG;
  const MlpPlan p = plan_mlp(M, xt, gate, down);
  if (ws_bytes < p.bytes) return W4A16_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(ws);
  if (p.mfma) {
    const int H = gate->K, I = gate->N;
    _Float16* apx = reinterpret_cast<_Float16*>(wsb + p.apx_off);
    float* rsx = reinterpret_cast<float*>(wsb + p.rsx_off);
    float* h = reinterpret_cast<float*>(wsb + p.h_off);
    _Float16* aph = reinterpret_cast<_Float16*>(wsb + p.aph_off);
    float* rsh = reinterpret_cast<float*>(wsb + p.rsh_off);
    EventMarks::Bracket b = ev.bracket();
    st = launch_mfma_prep(x, xt, M, p.gu.Mp, H, p.gu.P, nullptr, 0, nullptr, apx, rsx, stream, b.start, b.stop);
    if (st != W4A16_OK) return st;
    MfmaArgs a = mfma_dense_args(p.gu, M, gate, up, 1, apx, rsx, wsb, p.partials_off, p.counters_off);
    a.h = h;
    if (p.gu.S > 1) defer_split_k(a, p.gu);
    b = ev.bracket();
    st = launch_mfma(a, p.gu.P, p.gu.tasks * p.gu.S, stream, b.start, b.stop);
    if (st != W4A16_OK) return st;
    b = ev.bracket();
    if (p.split_pieces)  // h's pieces per down split, from the gate/up split sums
      st = launch_prep_split_pieces(a.planes, a.S, a.plane_rows, a.plane_ld, rsx, M, p.dn.Mp, I, p.dn.P,
                                    p.dn.gps * kGroup, aph, rsh, stream, b.start, b.stop);
    else if (p.gu.S > 1)  // h from the gate/up split sums, then its pieces
      st = launch_prep_planes(a.planes, a.S, a.plane_rows, a.plane_ld, rsx, M, p.dn.Mp, I, p.dn.P, h, aph, rsh,
                              stream, b.start, b.stop);
    else
      st = launch_mfma_prep(h, W4A16_F32, M, p.dn.Mp, I, p.dn.P, nullptr, 0, nullptr, aph, rsh, stream, b.start,
                            b.stop);
    if (st != W4A16_OK) return st;
    MfmaArgs d = mfma_dense_args(p.dn, M, down, nullptr, 0, aph, rsh, wsb, p.partials_off,
                                 p.counters_off);
    d.out = y;
    b = ev.bracket();
    if (p.dn.S == 1) return launch_mfma(d, p.dn.P, p.dn.tasks * p.dn.S, stream, b.start, b.stop);
    defer_split_k(d, p.dn);
    st = launch_mfma(d, p.dn.P, p.dn.tasks * p.dn.S, stream, b.start, b.stop);
    if (st != W4A16_OK) return st;
    b = ev.bracket();
    return launch_plane_sum(d.planes, d.S, d.plane_rows, d.plane_ld, rsh, p.split_pieces ? p.dn.Mp : 0, M, down->N,
                            y, stream, b.start, b.stop);
  }
  if (!counters_fit(p.tasks_gu, p.S_gu) || !counters_fit(p.tasks_d, p.S_d))
    return W4A16_ERR_UNSUPPORTED;
  float* h = reinterpret_cast<float*>(wsb + p.h_off);
  GemvArgs a = gemv_dense_args(M, gate, up, 1, x, xt == W4A16_BF16, gemv_pieces(xt), p.tiles_gu, p.S_gu, p.gps_gu,
                               wsb, p.partials_off, p.counters_off);
  a.h = h;
  EventMarks::Bracket b = ev.bracket();
  st = launch_gemv(a, p.tasks_gu * p.S_gu, stream, b.start, b.stop);
  if (st != W4A16_OK) return st;
  GemvArgs d = gemv_dense_args(M, down, nullptr, 0, h, false, gemv_pieces(xt), p.tiles_d, p.S_d, p.gps_d, wsb,
                               p.partials_off, p.counters_off);
  d.out = y;
  b = ev.bracket();
  return launch_gemv(d, p.tasks_d * p.S_d, stream, b.start, b.stop);
}
}  // namespace w4

extern "C" w4a16_status_t w4a16_swiglu_mlp(const void* x, w4a16_dtype_t xt, int32_t M,
                                           const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                           const w4a16_weight_t* down, float* y, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  EventMarks none;
  return swiglu_mlp_impl(x, xt, M, gate, up, down, y, ws, ws_bytes, stream, none);
}

extern "C" w4a16_status_t w4a16_swiglu_mlp_timed(const void* x, w4a16_dtype_t xt, int32_t M,
                                                 const w4a16_weight_t* gate,
                                                 const w4a16_weight_t* up,
                                                 const w4a16_weight_t* down, float* y, void* ws,
                                                 size_t ws_bytes, hipStream_t stream,
                                                 hipEvent_t* events, int32_t capacity,
                                                 int32_t* recorded) {
  if (capacity < 0 || (capacity > 0 && events == nullptr)) return W4A16_ERR_INVALID_ARG;
  EventMarks ev;
  ev.events = events;
  ev.capacity = capacity;
  w4a16_status_t st = swiglu_mlp_impl(x, xt, M, gate, up, down, y, ws, ws_bytes, stream, ev);
  if (recorded != nullptr) *recorded = ev.recorded;
  return st;
}

// ---------------------------------------------------------------- allocation-free entry point

namespace w4 {
namespace {

// The workspace of w4a16_swiglu_mlp_static: a static device array, one copy
// on every GPU the library runs on, held until the process ends.
__device__ __align__(256) unsigned char scratch[W4A16_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // the array's device address on each GPU (null: not set up)

// The device address of `scratch` on the current device, set up on the first
// call there: hipGetSymbolAddress with that device current (each GPU holds
// its own copy at its own address), then the split-K counters at its start
// are zeroed by a fill kernel on `stream` (every later call leaves them at
// zero again).  Host code uses only this address, never the array's name.
w4a16_status_t static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return W4A16_ERR_HIP;
  if (dev >= kMaxDevices) return W4A16_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return W4A16_ERR_HIP;
    const w4a16_status_t st = w4a16_workspace_init(p, kCounterBytes, stream);
    if (st != W4A16_OK) return st;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return W4A16_OK;
}

}  // namespace
}  // namespace w4

extern "C" w4a16_status_t w4a16_swiglu_mlp_static(const void* x, w4a16_dtype_t xt, int32_t M,
                                                  const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                                  const w4a16_weight_t* down, float* y, hipStream_t stream) {
  w4a16_status_t st = check_mlp(gate, up, down);
  if (st != W4A16_OK) return st;
  if (M < 0 || (xt != W4A16_F32 && xt != W4A16_BF16)) return W4A16_ERR_INVALID_ARG;
  if (M == 0 || gate->K == 0 || gate->N == 0) return W4A16_OK;
  if (x == nullptr || y == nullptr || !aligned16(x) || !aligned16(y)) return W4A16_ERR_INVALID_ARG;
  if (plan_mlp(M, xt, gate, down).bytes > W4A16_STATIC_SCRATCH_BYTES) return W4A16_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = static_scratch(stream, &ws)) != W4A16_OK) return st;
  EventMarks none;
  return swiglu_mlp_impl(x, xt, M, gate, up, down, y, ws, W4A16_STATIC_SCRATCH_BYTES, stream, none);
}
