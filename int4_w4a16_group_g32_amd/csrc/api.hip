// Host entry points: argument checks, workspace layout and kernel dispatch for
// the dense GEMM and the dense SwiGLU MLP.
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

GemmPlan plan_gemm(int M, const w4a16_weight_t* w, w4a16_dtype_t xt) {
  GemmPlan p;
  p.P = pieces_for(xt);
  const int G = w->K / kGroup;
  const size_t items = (static_cast<size_t>(M) + kMaxGemvRows - 1) / kMaxGemvRows;
  p.tiles = w->N / 64;
  p.tasks = items * p.tiles;
  p.S = gemv_splits(p.tasks, G);
  Carve c;
  c.take(p.counters_off, kCounterBytes);
  c.take(p.xq_off, static_cast<size_t>(M) * G * 8 * p.P * 4);
  c.take(p.xf_off, static_cast<size_t>(M) * G * 4);
  c.take(p.partials_off, gemv_partial_bytes(p.tasks, p.S));
  p.bytes = c.cursor;
  return p;
}

MlpPlan plan_mlp(int M, w4a16_dtype_t xt, const w4a16_weight_t* gate, const w4a16_weight_t* down) {
  MlpPlan p;
  p.P = pieces_for(xt);
  const int H = gate->K, I = gate->N;
  const int GH = H / kGroup, GI = I / kGroup;
  const size_t items = (static_cast<size_t>(M) + kMaxGemvRows - 1) / kMaxGemvRows;
  p.tiles_gu = I / 32;
  p.tasks_gu = items * p.tiles_gu;
  p.S_gu = gemv_splits(p.tasks_gu, GH);
  p.tiles_d = down->N / 64;
  p.tasks_d = items * p.tiles_d;
  p.S_d = gemv_splits(p.tasks_d, GI);
  Carve c;
  c.take(p.counters_off, kCounterBytes);
  c.take(p.xq_off, static_cast<size_t>(M) * GH * 8 * p.P * 4);
  c.take(p.xf_off, static_cast<size_t>(M) * GH * 4);
  c.take(p.hq_off, static_cast<size_t>(M) * GI * 8 * p.P * 4);
  c.take(p.hf_off, static_cast<size_t>(M) * GI * 4);
  const size_t part = std::max(gemv_partial_bytes(p.tasks_gu, p.S_gu),
                               gemv_partial_bytes(p.tasks_d, p.S_d));
  c.take(p.partials_off, part);
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
                         const int32_t* xq, const float* xf, int tiles, int S, char* ws,
                         size_t partials_off, size_t counters_off) {
  GemvArgs a{};
  a.xq = xq;
  a.xf = xf;
  a.G = w0->K / kGroup;
  a.R = M;
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
  a.gps = (a.G + S - 1) / S;
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

extern "C" w4a16_status_t w4a16_gemm(const void* x, w4a16_dtype_t xt, int32_t M,
                                     const w4a16_weight_t* w, float* y, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
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
  if (!counters_fit(p.tasks, p.S)) return W4A16_ERR_UNSUPPORTED;
  char* wsb = static_cast<char*>(ws);
  int32_t* xq = reinterpret_cast<int32_t*>(wsb + p.xq_off);
  float* xf = reinterpret_cast<float*>(wsb + p.xf_off);
  st = launch_prep_pieces(x, xt, M, w->K, p.P, nullptr, 0, xq, xf, stream);
  if (st != W4A16_OK) return st;
  GemvArgs a = gemv_dense_args(M, w, nullptr, 0, xq, xf, p.tiles, p.S, wsb, p.partials_off,
                               p.counters_off);
  a.out = y;
  return launch_gemv(a, p.P, p.tasks * p.S, stream);
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
  if (!counters_fit(p.tasks_gu, p.S_gu) || !counters_fit(p.tasks_d, p.S_d))
    return W4A16_ERR_UNSUPPORTED;
  char* wsb = static_cast<char*>(ws);
  int32_t* xq = reinterpret_cast<int32_t*>(wsb + p.xq_off);
  float* xf = reinterpret_cast<float*>(wsb + p.xf_off);
  int32_t* hq = reinterpret_cast<int32_t*>(wsb + p.hq_off);
  float* hf = reinterpret_cast<float*>(wsb + p.hf_off);
  if ((st = ev.mark(stream)) != W4A16_OK) return st;
  st = launch_prep_pieces(x, xt, M, gate->K, p.P, nullptr, 0, xq, xf, stream);
  if (st != W4A16_OK) return st;
  GemvArgs a = gemv_dense_args(M, gate, up, 1, xq, xf, p.tiles_gu, p.S_gu, wsb, p.partials_off,
                               p.counters_off);
  a.hq = hq;
  a.hf = hf;
  if ((st = ev.mark(stream)) != W4A16_OK) return st;
  st = launch_gemv(a, p.P, p.tasks_gu * p.S_gu, stream);
  if (st != W4A16_OK) return st;
  GemvArgs d = gemv_dense_args(M, down, nullptr, 0, hq, hf, p.tiles_d, p.S_d, wsb, p.partials_off,
                               p.counters_off);
  d.out = y;
  if ((st = ev.mark(stream)) != W4A16_OK) return st;
  st = launch_gemv(d, p.P, p.tasks_d * p.S_d, stream);
  if (st != W4A16_OK) return st;
  return ev.mark(stream);
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
