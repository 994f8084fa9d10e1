// Workspace plans and shared host helpers of the entry points (internal).
#pragma once

#include <algorithm>

#include "gemv.h"
#include "mfma.h"

namespace w4 {

// Split-K arrival counters sit at the start of every workspace.
constexpr size_t kCounterBytes = 64 * 1024;

struct Carve {
  size_t cursor = 0;
  void take(size_t& off, size_t bytes);
};

// MFMA path (rows above the GEMV range)
struct MfmaPlan {
  bool wide = false;  // wide tiles (256 x 128) instead of 64 x 256
  int P = 0, Mp = 0, tiles = 0, S = 1, gps = 0;
  size_t items = 0, tasks = 0;
};
// allow_wide: the caller launches wide tiles when the plan says so
MfmaPlan plan_mfma(int rows, int N, int mode, int K, w4a16_dtype_t xt, bool allow_wide);

struct GemmPlan {
  int S = 1, gps = 1;
  int tiles = 0;
  size_t tasks = 0;
  size_t counters_off = 0, partials_off = 0;
  bool mfma = false;
  MfmaPlan mf;
  size_t ap_off = 0, rs_off = 0;
  size_t bytes = 0;
};

struct MlpPlan {
  int tiles_gu = 0, S_gu = 1, gps_gu = 1, tiles_d = 0, S_d = 1, gps_d = 1;
  size_t tasks_gu = 0, tasks_d = 0;
  size_t counters_off = 0, h_off = 0, partials_off = 0;
  // MFMA path
  bool mfma = false;
  MfmaPlan gu, dn;
  size_t apx_off = 0, rsx_off = 0, aph_off = 0, rsh_off = 0;
  bool split_pieces = false;  // h pieces per down K split (rsh: [S_down][Mp])
  size_t bytes = 0;
};

// Optional measurement hook: hands out caller events in pairs, the start and
// stop of each kernel an entry point launches (taken by the runtime from the
// kernel's own dispatch).
struct EventMarks {
  hipEvent_t* events = nullptr;
  int capacity = 0;
  int recorded = 0;
  // The start and stop events of the next kernel (both null once the caller's
  // array is used up, or without events).
  struct Bracket {
    hipEvent_t start = nullptr, stop = nullptr;
  };
  Bracket bracket() {
    Bracket b;
    if (events != nullptr && recorded + 2 <= capacity) {
      b.start = events[recorded++];
      b.stop = events[recorded++];
    }
    return b;
  }
};

size_t gemv_partial_bytes(size_t tasks, int S);
GemmPlan plan_gemm(int M, const w4a16_weight_t* w, w4a16_dtype_t xt);
MlpPlan plan_mlp(int M, w4a16_dtype_t xt, const w4a16_weight_t* gate, const w4a16_weight_t* down);
bool counters_fit(size_t tasks, int S);
w4a16_status_t check_dense_grouped(const w4a16_weight_t* w);
w4a16_status_t check_mlp(const w4a16_weight_t* gate, const w4a16_weight_t* up,
                         const w4a16_weight_t* down);
bool ranges_overlap(const void* a, size_t abytes, const void* b, size_t bbytes);
size_t dtype_bytes(w4a16_dtype_t xt);
// pieces: gemv_pieces of the layer's activation type (the float32
// intermediate of a bf16 layer takes one piece, as its rows do)
GemvArgs gemv_dense_args(int M, const w4a16_weight_t* w0, const w4a16_weight_t* w1, int mode,
                         const void* x, bool x_bf16, int pieces, int tiles, int S, int gps, char* ws,
                         size_t partials_off, size_t counters_off);

}  // namespace w4
