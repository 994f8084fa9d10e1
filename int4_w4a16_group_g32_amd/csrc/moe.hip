// Routed-expert MoE layer: expert grouping of (token, slot) pairs, grouped
// W4A16 GEMVs over the ragged per-expert row lists and the weighted combine.
//
// Page "The Final Wire: How a Single Edit Integrated INT4 Quantization into a
// Native DDTree Inference Engine", section "What the Edit Actually Changes":
// the router selects top-k experts per token and each selected expert runs its
// own gate, up and down projections through the W4A16 path.  Per-expert row
// counts are produced and consumed on the device only.
#include <climits>

#include "dispatch.h"

#include <hip/hip_ext.h>

namespace w4 {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kSharedGemvRows = 64;
#ifndef W4_SHARED_FIRST
#define W4_SHARED_FIRST 1
#endif
constexpr bool kSharedFirst = W4_SHARED_FIRST != 0;  // shared expert's items ahead of the routed ones
#ifndef W4_COMBINE_BATCH
#define W4_COMBINE_BATCH 8
#endif
constexpr int kCombineBatch = W4_COMBINE_BATCH;  // routed slots whose loads the combine issues together
#ifndef W4_GEMV_EXPERT_ROWS_BF16
#define W4_GEMV_EXPERT_ROWS_BF16 16
#endif
// Experts with at most this many rows run on the GEMV (as items of
// gemv_rows(xt) rows each), heavier ones on the MFMA tiles.
inline int gemv_expert_rows(w4a16_dtype_t xt) {
  return xt == W4A16_BF16 ? W4_GEMV_EXPERT_ROWS_BF16 : kMaxGemvRows;
}
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRouteLdsInts = 12288;  // 48 KiB: per-wave expert counts and totals
constexpr int kRouteChunk = 8;       // 64-pair steps whose ids one wave loads together

// Waves that place pairs for E experts: each keeps E counters in LDS, next to
// one row of per-expert totals.
__host__ __device__ inline int route_waves(int E) {
  const int w = kRouteLdsInts / E - 1;
  return w < 1 ? 1 : (w > kRouteWaves ? kRouteWaves : w);
}

// Inclusive scan of v over the block's threads in thread order: a shuffle
// scan within each wave, then over the wave totals (wsum, kRouteWaves
// entries).  Every thread calls it; it begins and ends with a barrier, so
// back-to-back calls may reuse wsum.
__device__ __forceinline__ int block_scan_incl(int v, int* wsum) {
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid % kWave, wv = tid / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  __syncthreads();
  if (lane == kWave - 1) wsum[wv] = v;
  __syncthreads();
  if (wv == 0) {
    int s = lane < kRouteWaves ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < kRouteWaves; off <<= 1) {
      const int t = __shfl_up(s, off);
      if (lane >= off) s += t;
    }
    if (lane < kRouteWaves) wsum[lane] = s;
  }
  __syncthreads();
  return wv > 0 ? v + wsum[wv - 1] : v;
}

// Lanes of this wave whose key equals this lane's key (keys < 2^bits): one
// ballot per key bit, intersected.
__device__ __forceinline__ uint64_t same_key_lanes(int key, int bits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < bits; ++b) {
    const bool on = (key >> b) & 1;
    const uint64_t v = __ballot(on);
    m &= on ? v : ~v;
  }
  return m;
}

// Stable counting sort of pairs p = t * top_k + slot by expert id, in one
// workgroup.  Wave w of the W placing waves owns the pairs [w L, (w + 1) L);
// pass A counts each wave's pairs per expert, a scan along waves per expert
// (after the scan over experts) gives every wave its first position per
// expert, and pass B places the pairs: a lane's position is its wave's
// running position for its expert plus the number of lower lanes in the same
// 64-pair step with the same expert, so the order within an expert is pair
// order.  Ids outside [0, E) are skipped (inv = -1).  Optionally also emits
// the work items of the grouped layer: an expert with at most expert_rows
// rows is cut into GEMV items of gemv_rows rows (8 for float32 activations,
// 16 for bf16), a heavier one into MFMA items of kMfmaRows rows, and
// heavy[pos] marks the positions that belong to MFMA items.  With
// shared_rows = M a shared expert (id E) takes the positions M * top_k + t,
// t = 0 .. M-1, one per token in token order (gather entry t * top_k): up to
// kSharedGemvRows rows as GEMV items of kMaxGemvRows rows, which join the
// routed experts' GEMV launches (the MFMA items have no K split, so a lone
// heavy expert would be a long serial tail), more as MFMA items; either way
// they take the first item indices of their launch.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const int32_t* __restrict__ ids, int M, int top_k, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ inv,
    int4* __restrict__ items_g, int4* __restrict__ items_m, int32_t* __restrict__ n_items,
    int32_t* __restrict__ heavy, int shared_rows, int gemv_rows, int expert_rows) {
  extern __shared__ int lds[];  // wc[W][E], then tot[E]
  __shared__ int carry;
  __shared__ int any_mfma;  // some expert has more than expert_rows rows
  __shared__ int wsum[kRouteWaves];
  const int tid = threadIdx.x;
  const int W = route_waves(E);
  int* wc = lds;
  int* tot = lds + W * E;
  const int pairs = M * top_k;
  const int L = (pairs + W - 1) / W;
  int bits = 1;
  while ((1 << bits) <= E) ++bits;  // keys 0 .. E (E = skipped)
  const int wv = tid / kWave, lane = tid % kWave;
  const uint64_t below = (1ull << lane) - 1;

  for (int i = tid; i < (W + 1) * E; i += kRouteThreads) lds[i] = 0;
  if (tid == 0) any_mfma = 0;
  __syncthreads();
  // The keys of a wave's pairs are read kRouteChunk steps of 64 at a time,
  // all loads in flight together, instead of one dependent load per step.
  auto load_keys = [&](int c0, int p1, int key[kRouteChunk]) {
#pragma unroll
    for (int j = 0; j < kRouteChunk; ++j) {
      const int p = c0 + j * kWave + lane;
      const int e = p < p1 ? ids[p] : E;
      key[j] = (e >= 0 && e < E) ? e : E;
    }
  };
  // A. per-wave counts
  if (wv < W) {
    const int p0 = wv * L, p1 = min(pairs, p0 + L);
    for (int c0 = p0; c0 < p1; c0 += kRouteChunk * kWave) {
      int key[kRouteChunk];
      load_keys(c0, p1, key);
#pragma unroll
      for (int j = 0; j < kRouteChunk; ++j) {
        if (c0 + j * kWave >= p1) break;  // (wave-uniform)
        const uint64_t m = same_key_lanes(key[j], bits);
        if ((m & below) == 0 && key[j] < E) wc[wv * E + key[j]] += __popcll(m);
      }
    }
  }
  __syncthreads();
  // totals per expert
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < W; ++w) run += wc[w * E + e];
    tot[e] = run;
    counts[e] = run;
    if (run > expert_rows) any_mfma = 1;
  }
  __syncthreads();
  // offsets = exclusive scan of the totals (blocks of kRouteThreads, serial carry)
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < E; base += kRouteThreads) {
    const int e = base + tid;
    const int v = e < E ? tot[e] : 0;
    const int incl = block_scan_incl(v, wsum);
    if (e < E) {
      offsets[e] = carry + incl - v;
      tot[e] = carry + incl - v;
    }
    __syncthreads();
    if (tid == kRouteThreads - 1) carry += incl;
    __syncthreads();
  }
  if (tid == 0) offsets[E] = carry;
  // first position of every wave per expert
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = tot[e];
    for (int w = 0; w < W; ++w) {
      const int t = wc[w * E + e];
      wc[w * E + e] = run;
      run += t;
    }
  }
  __syncthreads();
  // B. placement
  if (wv < W) {
    const int p0 = wv * L, p1 = min(pairs, p0 + L);
    for (int c0 = p0; c0 < p1; c0 += kRouteChunk * kWave) {
      int key[kRouteChunk];
      load_keys(c0, p1, key);
#pragma unroll
      for (int j = 0; j < kRouteChunk; ++j) {
        if (c0 + j * kWave >= p1) break;  // (wave-uniform)
        const int p = c0 + j * kWave + lane;
        const uint64_t m = same_key_lanes(key[j], bits);
        if (key[j] < E) {
          const int pos = wc[wv * E + key[j]] + __popcll(m & below);
          sorted_pairs[pos] = p;
          inv[p] = pos;
          if (heavy != nullptr) {
            // the expert's row count from the offsets in LDS (no global load per step)
            const int cnt = (key[j] + 1 < E ? tot[key[j] + 1] : carry) - tot[key[j]];
            heavy[pos] = cnt > expert_rows ? 1 : 0;
          }
        } else if (p < p1) {
          inv[p] = -1;
        }
        __builtin_amdgcn_wave_barrier();
        if ((m & below) == 0 && key[j] < E) wc[wv * E + key[j]] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  // the shared expert's positions follow the routed pairs
  for (int t = tid; t < shared_rows; t += kRouteThreads) {
    sorted_pairs[pairs + t] = t * top_k;
    if (heavy != nullptr) heavy[pairs + t] = shared_rows > kSharedGemvRows ? 1 : 0;
  }
  if (items_g == nullptr) return;
  __syncthreads();
  // C. work items: exclusive scans over experts of the GEMV and MFMA item counts.
  // The shared expert's items (all of one kind) take the first indices of
  // their launch, so they are dispatched first and the routed experts' items
  // fill in behind them.  MFMA items are laid out longest first: every full
  // 64-row item (expert order), then the experts' partial last items with 33
  // to 63 rows, 17 to 32 and 1 to 16, so the cheap items (whose row blocks
  // without rows skip their MFMAs) run in the launch's last, partly filled
  // round of workgroups.
  const int shared_kind = shared_rows > kSharedGemvRows ? 1 : 0;
  const int shared_step = shared_kind == 1 ? kMfmaRows : kMaxGemvRows;
  const int shared_items = (shared_rows + shared_step - 1) / shared_step;
  // pass 0: GEMV items; 1: full MFMA items; 2, 3, 4: partial MFMA items by
  // row class
  for (int pass = 0; pass < 5; ++pass) {
    const int kind = pass == 0 ? 0 : 1;
    if (pass == 1 && any_mfma == 0) {  // no MFMA items but the shared expert's
      if (tid == 0) n_items[1] = shared_kind == 1 ? shared_items : 0;
      break;
    }
    if (pass < 2) {
      const int lead = (kSharedFirst && kind == shared_kind) ? shared_items : 0;
      if (tid == 0) carry = lead;
    }
    __syncthreads();
    for (int base = 0; base < E; base += kRouteThreads) {
      const int e = base + tid;
      const int c0 = e < E ? counts[e] : 0;
      const int rem = c0 % kMfmaRows;
      int n = 0;
      if (kind == 0) {
        n = (c0 > 0 && c0 <= expert_rows) ? (c0 + gemv_rows - 1) / gemv_rows : 0;
      } else if (c0 > expert_rows) {
        if (pass == 1) n = c0 / kMfmaRows;
        else if (pass == 2) n = rem > 32 ? 1 : 0;
        else if (pass == 3) n = rem > 16 && rem <= 32 ? 1 : 0;
        else n = rem > 0 && rem <= 16 ? 1 : 0;
      }
      const int incl = block_scan_incl(n, wsum);
      if (n > 0) {
        int it = carry + incl - n;
        const int o0 = offsets[e];
        if (kind == 0) {
          for (int r = 0; r < c0; r += gemv_rows, ++it)
            items_g[it] = make_int4(e, o0 + r, min(gemv_rows, c0 - r), 0);
        } else if (pass == 1) {
          for (int r = 0; r + kMfmaRows <= c0; r += kMfmaRows, ++it)
            items_m[it] = make_int4(e, o0 + r, kMfmaRows, 0);
        } else {
          items_m[it] = make_int4(e, o0 + c0 - rem, rem, 0);
        }
      }
      __syncthreads();
      if (tid == kRouteThreads - 1) carry += incl;
      __syncthreads();
    }
    if ((pass == 0 || pass == 4) && tid == 0)
      n_items[kind] = carry + ((!kSharedFirst && kind == shared_kind) ? shared_items : 0);
    __syncthreads();
  }
  if (shared_rows > 0 && tid == 0) {
    int it = kSharedFirst ? 0 : n_items[shared_kind] - shared_items;
    int4* dst = shared_kind == 1 ? items_m : items_g;
    for (int r = 0; r < shared_rows; r += shared_step, ++it)
      dst[it] = make_int4(E, pairs + r, min(shared_step, shared_rows - r), 0);
  }
}

// y[t][n] = sum over slots, in slot order, of w[t][s] * o[inv[t*top_k+s]][n].
// A thread produces four consecutive columns (16-byte loads and stores of
// float32 o, 8-byte loads of bf16 o; H is a multiple of 32).
// With shared0 >= 0 the shared expert's output row o[shared0 + t] is added
// last, with weight 1.
__device__ __forceinline__ float4 load_o4(const float* o, size_t at) {
  return *reinterpret_cast<const float4*>(o + at);
}
__device__ __forceinline__ float4 load_o4(const uint16_t* o, size_t at) {
  const uint2 b = *reinterpret_cast<const uint2*>(o + at);
  return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u), __uint_as_float(b.y << 16),
                     __uint_as_float(b.y & 0xffff0000u));
}

template <typename OT>
__global__ void combine_kernel(const OT* __restrict__ o, const int32_t* __restrict__ inv,
                               const float* __restrict__ topk_w, int M, int top_k, int H, int shared0,
                               float* __restrict__ y) {
  const int H4 = H / 4;
  const size_t idx = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (idx >= static_cast<size_t>(M) * H4) return;
  const int t = static_cast<int>(idx / H4);
  const int n4 = static_cast<int>(idx % H4);
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  // Slots in batches of kCombineBatch: all loads of a batch are issued before
  // its first fma (a skipped slot reads row 0 and leaves acc unchanged), and
  // the fmas run in slot order.
  for (int s0 = 0; s0 < top_k; s0 += kCombineBatch) {
    int pos[kCombineBatch];
    float w[kCombineBatch];
    float4 v[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int s = s0 + i;
      pos[i] = s < top_k ? inv[t * top_k + s] : -1;
      w[i] = s < top_k ? topk_w[t * top_k + s] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i)
      v[i] = load_o4(o, static_cast<size_t>(pos[i] < 0 ? 0 : pos[i]) * H + 4 * static_cast<size_t>(n4));
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      if (pos[i] < 0) continue;
      acc.x = fmaf(w[i], v[i].x, acc.x);
      acc.y = fmaf(w[i], v[i].y, acc.y);
      acc.z = fmaf(w[i], v[i].z, acc.z);
      acc.w = fmaf(w[i], v[i].w, acc.w);
    }
  }
  if (shared0 >= 0) {
    const float4 v = load_o4(o, static_cast<size_t>(shared0 + t) * H + 4 * static_cast<size_t>(n4));
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  reinterpret_cast<float4*>(y + static_cast<size_t>(t) * H)[n4] = acc;
}

size_t route_lds_bytes(int E) { return static_cast<size_t>(route_waves(E) + 1) * E * sizeof(int); }

w4a16_status_t launch_route(const int32_t* ids, int M, int top_k, int E, int32_t* counts,
                            int32_t* offsets, int32_t* sorted_pairs, int32_t* inv, int4* items_g,
                            int4* items_m, int32_t* n_items, int32_t* heavy, int shared_rows,
                            int gemv_rows, int expert_rows, hipStream_t stream, hipEvent_t start = nullptr,
                            hipEvent_t stop = nullptr) {
  if (2 * E > kRouteLdsInts) return W4A16_ERR_UNSUPPORTED;
  const size_t lds = route_lds_bytes(E);
  hipExtLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), lds, stream, start, stop, 0, ids, M, top_k, E,
                        counts, offsets, sorted_pairs, inv, items_g, items_m, n_items, heavy, shared_rows, gemv_rows,
                        expert_rows);
  return launch_status();
}

struct MoePlan {
  int P = 0, Mp = 0;
  size_t pairs = 0, max_items = 0, max_mitems = 0;
  size_t positions = 0;  // pairs, then one per token for a shared expert
  size_t counts_off, offsets_off, sorted_off, inv_off, items_off, mitems_off, nitems_off, heavy_off;
  size_t h_off, o_off;
  size_t apx_off, rsx_off, aph_off, rsh_off;
  bool mfma = false;  // some expert can have more than gemv_expert_rows(xt) rows
  int expert_rows = 0;  // experts above this many rows run on MFMA items
  size_t bytes = 0;
};

MoePlan plan_moe(int M, int top_k, w4a16_dtype_t xt, const w4a16_weight_t* gate, bool shared) {
  MoePlan p;
  p.P = mfma_pieces(xt);
  const int E = gate->num_experts, H = gate->K, I = gate->N;
  p.pairs = static_cast<size_t>(M) * top_k;
  p.positions = p.pairs + (shared ? static_cast<size_t>(M) : 0);
  // An expert gets at most M rows while a token's ids are distinct.  Without
  // an MFMA launch every expert is cut into GEMV items, so that ids repeated
  // within a token (more rows than M for one expert) still have their items.
  p.mfma = M > gemv_expert_rows(xt);
  p.expert_rows = p.mfma ? gemv_expert_rows(xt) : INT_MAX;
  if (p.mfma) {
    // light experts: at most gemv_expert_rows rows, in items of gemv_rows rows
    const int per_expert = (gemv_expert_rows(xt) + gemv_rows(xt) - 1) / gemv_rows(xt);
    p.max_items = std::min<size_t>(E, p.pairs) * per_expert + 1;
  } else {
    p.max_items = p.pairs / gemv_rows(xt) + std::min<size_t>(E, p.pairs) + 1;
  }
  p.max_mitems =
      p.mfma ? p.pairs / kMfmaRows + std::min<size_t>(E, p.pairs / (gemv_expert_rows(xt) + 1)) + 1 : 0;
  if (shared) {  // the shared expert is one more expert with M rows
    if (M <= kSharedGemvRows)
      p.max_items += (static_cast<size_t>(M) + kMaxGemvRows - 1) / kMaxGemvRows;
    else
      p.max_mitems += (static_cast<size_t>(M) + kMfmaRows - 1) / kMfmaRows;
  }
  p.Mp = p.mfma ? mfma_rows_padded(static_cast<int>(p.positions)) : 0;
  Carve c;
  size_t dummy;
  c.take(dummy, kCounterBytes);
  c.take(p.counts_off, static_cast<size_t>(E) * 4);
  c.take(p.offsets_off, static_cast<size_t>(E + 1) * 4);
  c.take(p.sorted_off, p.positions * 4);
  c.take(p.inv_off, p.pairs * 4);
  c.take(p.items_off, p.max_items * 16);
  c.take(p.mitems_off, std::max<size_t>(p.max_mitems, 1) * 16);
  c.take(p.nitems_off, 16);
  c.take(p.heavy_off, p.positions * 4);
  c.take(p.h_off, std::max<size_t>(p.positions, p.Mp) * I * (xt == W4A16_BF16 ? 2 : 4));  // bf16 for bf16 x
  c.take(p.o_off, p.positions * H * (xt == W4A16_BF16 ? 2 : 4));  // per-pair outputs: bf16 for bf16 x
  // activation pieces: one row per token (the tiles map positions to tokens)
  const size_t xrows = p.mfma ? static_cast<size_t>(M) : 0;
  c.take(p.apx_off, static_cast<size_t>(p.P) * xrows * H * 2);
  c.take(p.rsx_off, xrows * 4);
  c.take(p.aph_off, static_cast<size_t>(p.P) * p.Mp * I * 2);
  c.take(p.rsh_off, static_cast<size_t>(p.Mp) * 4);
  p.bytes = c.cursor;
  return p;
}

w4a16_status_t check_moe(const w4a16_weight_t* gate, const w4a16_weight_t* up,
                         const w4a16_weight_t* down) {
  const w4a16_weight_t* ws[3] = {gate, up, down};
  for (const w4a16_weight_t* w : ws) {
    w4a16_status_t st = check_weight(w);
    if (st != W4A16_OK) return st;
    if (w->layout != W4A16_LAYOUT_GROUPED) return W4A16_ERR_UNSUPPORTED;
  }
  if (gate->num_experts != up->num_experts || gate->num_experts != down->num_experts)
    return W4A16_ERR_UNSUPPORTED;
  if (gate->K != up->K || gate->N != up->N) return W4A16_ERR_UNSUPPORTED;
  if (gate->group_size != up->group_size) return W4A16_ERR_UNSUPPORTED;  // one launch streams both
  if (down->K != gate->N || down->N != gate->K) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

// A shared expert: one SwiGLU MLP of the routed experts' shapes and group sizes, GROUPED.
w4a16_status_t check_shared(const w4a16_weight_t* gate, const w4a16_weight_t* down, const w4a16_weight_t* sg,
                            const w4a16_weight_t* su, const w4a16_weight_t* sd) {
  const w4a16_status_t st = check_moe(sg, su, sd);
  if (st != W4A16_OK) return st;
  if (sg->num_experts != 1) return W4A16_ERR_UNSUPPORTED;
  if (sg->K != gate->K || sg->N != gate->N) return W4A16_ERR_UNSUPPORTED;
  if (sg->group_size != gate->group_size || sd->group_size != down->group_size) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

}  // namespace
}  // namespace w4

using namespace w4;

extern "C" w4a16_status_t w4a16_moe_route(const int32_t* topk_ids, int32_t M, int32_t top_k,
                                          int32_t E, int32_t* counts, int32_t* offsets,
                                          int32_t* sorted_pairs, int32_t* inv,
                                          hipStream_t stream) {
  if (M < 0 || E < 1 || top_k < 1 || top_k > E) return W4A16_ERR_INVALID_ARG;
  if (counts == nullptr || offsets == nullptr) return W4A16_ERR_INVALID_ARG;
  if (!aligned16(counts) || !aligned16(offsets)) return W4A16_ERR_INVALID_ARG;
  if (M > 0) {
    if (topk_ids == nullptr || sorted_pairs == nullptr || inv == nullptr) return W4A16_ERR_INVALID_ARG;
    if (!aligned16(topk_ids) || !aligned16(sorted_pairs) || !aligned16(inv))
      return W4A16_ERR_INVALID_ARG;
  }
  return launch_route(topk_ids, M, top_k, E, counts, offsets, sorted_pairs, inv, nullptr, nullptr,
                      nullptr, nullptr, 0, kMaxGemvRows, kMaxGemvRows, stream);
}

extern "C" size_t w4a16_moe_workspace_bytes(int32_t M, int32_t top_k, w4a16_dtype_t xt,
                                            const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                            const w4a16_weight_t* down) {
  if (M <= 0 || top_k < 1 || check_moe(gate, up, down) != W4A16_OK) return 0;
  if (xt != W4A16_F32 && xt != W4A16_BF16) return 0;
  return plan_moe(M, top_k, xt, gate, false).bytes;
}

extern "C" size_t w4a16_moe_shared_workspace_bytes(int32_t M, int32_t top_k, w4a16_dtype_t xt,
                                                   const w4a16_weight_t* gate, const w4a16_weight_t* up,
                                                   const w4a16_weight_t* down,
                                                   const w4a16_weight_t* shared_gate,
                                                   const w4a16_weight_t* shared_up,
                                                   const w4a16_weight_t* shared_down) {
  if (M <= 0 || top_k < 1 || check_moe(gate, up, down) != W4A16_OK) return 0;
  if (check_shared(gate, down, shared_gate, shared_up, shared_down) != W4A16_OK) return 0;
  if (xt != W4A16_F32 && xt != W4A16_BF16) return 0;
  return plan_moe(M, top_k, xt, gate, true).bytes;
}

namespace w4 {
// sg, su, sd: the shared expert's gate, up and down (all null: none).
static w4a16_status_t moe_impl(const void* x, w4a16_dtype_t xt, int32_t M, const int32_t* topk_ids,
                               const float* topk_w, int32_t top_k, const w4a16_weight_t* gate,
                               const w4a16_weight_t* up, const w4a16_weight_t* down,
                               const w4a16_weight_t* sg, const w4a16_weight_t* su, const w4a16_weight_t* sd,
                               float* y, void* ws, size_t ws_bytes, hipStream_t stream, EventMarks& ev) {
  w4a16_status_t st = check_moe(gate, up, down);
  if (st != W4A16_OK) return st;
  const bool shared = sg != nullptr;
  if (shared && (st = check_shared(gate, down, sg, su, sd)) != W4A16_OK) return st;
  const int E = gate->num_experts, H = gate->K, I = gate->N;
  if (M < 0 || top_k < 1 || top_k > E || (xt != W4A16_F32 && xt != W4A16_BF16))
    return W4A16_ERR_INVALID_ARG;
  if (M == 0 || H == 0 || I == 0) return W4A16_OK;
  if (x == nullptr || topk_ids == nullptr || topk_w == nullptr || y == nullptr || ws == nullptr)
    return W4A16_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(y) ||
      !aligned16(ws))
    return W4A16_ERR_INVALID_ARG;
  if (ranges_overlap(x, static_cast<size_t>(M) * H * dtype_bytes(xt), y,
                     static_cast<size_t>(M) * H * 4))
    return W4A16_ERR_INVALID_ARG;
  const MoePlan p = plan_moe(M, top_k, xt, gate, shared);
  if (ws_bytes < p.bytes) return W4A16_ERR_WORKSPACE;
  char* b = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(b + p.counts_off);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + p.offsets_off);
  int32_t* sorted = reinterpret_cast<int32_t*>(b + p.sorted_off);
  int32_t* inv = reinterpret_cast<int32_t*>(b + p.inv_off);
  int4* items = reinterpret_cast<int4*>(b + p.items_off);
  int4* mitems = reinterpret_cast<int4*>(b + p.mitems_off);
  int32_t* n_items = reinterpret_cast<int32_t*>(b + p.nitems_off);
  int32_t* heavy = reinterpret_cast<int32_t*>(b + p.heavy_off);
  float* hraw = reinterpret_cast<float*>(b + p.h_off);
  float* o = reinterpret_cast<float*>(b + p.o_off);
  const int R = static_cast<int>(p.pairs);
  const int T = static_cast<int>(p.positions);  // routed pairs, then the shared expert's rows

  // 1. expert grouping and work items
  EventMarks::Bracket bk = ev.bracket();
  st = launch_route(topk_ids, M, top_k, E, counts, offsets, sorted, inv, items, mitems, n_items,
                    heavy, shared ? M : 0, gemv_rows(xt), p.expert_rows, stream, bk.start, bk.stop);
  if (st != W4A16_OK) return st;

  // 2. gate/up with the SwiGLU epilogue: light experts on the GEMV, heavy on MFMA tiles
  GemvArgs a{};
  a.x = x;
  a.x_bf16 = xt == W4A16_BF16 ? 1 : 0;
  a.pieces = gemv_pieces(xt);
  a.gather = sorted;
  a.top_k = top_k;
  a.G = H / kGroup;
  a.K = H;
  a.qw0 = reinterpret_cast<const u32x4*>(gate->qw);
  a.sc0 = gate->scales;
  a.qw1 = reinterpret_cast<const u32x4*>(up->qw);
  a.sc1 = up->scales;
  a.expert_stride = static_cast<size_t>(H / kGroup) * I;
  a.gshift = group_shift(gate);
  a.N = I;
  a.tiles = gemv_shape(p.max_items, I, 1, H / kGroup, 0).tiles;
  a.S = 1;
  a.gps = a.G;
  a.dense_rows = 0;
  a.items = items;
  a.n_items = n_items;
  a.mode = 1;
  a.h = hraw;
  a.h_bf16 = xt == W4A16_BF16;
  if (shared) {
    a.extra_plus1 = E + 1;
    a.qw0x = reinterpret_cast<const u32x4*>(sg->qw);
    a.sc0x = sg->scales;
    a.qw1x = reinterpret_cast<const u32x4*>(su->qw);
    a.sc1x = su->scales;
  }
  bk = ev.bracket();
  st = launch_gemv(a, p.max_items * a.tiles, stream, bk.start, bk.stop);
  if (st != W4A16_OK) return st;

  _Float16* apx = reinterpret_cast<_Float16*>(b + p.apx_off);
  float* rsx = reinterpret_cast<float*>(b + p.rsx_off);
  _Float16* aph = reinterpret_cast<_Float16*>(b + p.aph_off);
  float* rsh = reinterpret_cast<float*>(b + p.rsh_off);
  MfmaArgs ma{};
  if (p.mfma) {
    bk = ev.bracket();
    // pieces once per token; the tiles read position p from token sorted[p] / top_k
    st = launch_mfma_prep(x, xt, M, M, H, p.P, nullptr, 0, nullptr, apx, rsx, stream, bk.start, bk.stop);
    if (st != W4A16_OK) return st;
    ma.ap = apx;
    ma.rs = rsx;
    ma.Mp = M;
    ma.arow = sorted;
    ma.arow_div = top_k;
    ma.arow_n = T;
    ma.K = H;
    ma.G = H / kGroup;
    ma.qw0 = a.qw0;
    ma.sc0 = a.sc0;
    ma.qw1 = a.qw1;
    ma.sc1 = a.sc1;
    ma.expert_stride = a.expert_stride;
    ma.gshift = a.gshift;
    ma.N = I;
    ma.tiles = (I + kMfmaCols / 2 - 1) / (kMfmaCols / 2);
    ma.S = 1;
    ma.gps = ma.G;
    ma.dense_rows = 0;
    ma.items = mitems;
    ma.n_items = n_items + 1;
    ma.mode = 1;
    ma.h = hraw;
    ma.h_bf16 = xt == W4A16_BF16;
    ma.extra_plus1 = a.extra_plus1;
    ma.qw0x = a.qw0x;
    ma.sc0x = a.sc0x;
    ma.qw1x = a.qw1x;
    ma.sc1x = a.sc1x;
    bk = ev.bracket();
    st = launch_mfma(ma, p.P, p.max_mitems * ma.tiles, stream, bk.start, bk.stop);
    if (st != W4A16_OK) return st;
  }

  // 3. down projection into per-pair outputs
  GemvArgs d{};
  d.x = hraw;
  d.x_bf16 = xt == W4A16_BF16;
  d.pieces = gemv_pieces(xt);  // the items hold up to gemv_rows(xt) rows
  d.G = I / kGroup;
  d.K = I;
  d.qw0 = reinterpret_cast<const u32x4*>(down->qw);
  d.sc0 = down->scales;
  d.expert_stride = static_cast<size_t>(I / kGroup) * H;
  d.gshift = group_shift(down);
  d.N = H;
  d.tiles = gemv_shape(p.max_items, H, 0, I / kGroup, 0).tiles;
  d.S = 1;
  d.gps = d.G;
  d.dense_rows = 0;
  d.items = items;
  d.n_items = n_items;
  d.mode = 0;
  d.out = o;
  d.out_bf16 = xt == W4A16_BF16;
  if (shared) {
    d.extra_plus1 = E + 1;
    d.qw0x = reinterpret_cast<const u32x4*>(sd->qw);
    d.sc0x = sd->scales;
  }
  bk = ev.bracket();
  st = launch_gemv(d, p.max_items * d.tiles, stream, bk.start, bk.stop);
  if (st != W4A16_OK) return st;
  if (p.mfma) {
    bk = ev.bracket();
    st = launch_mfma_prep(hraw, xt, T, p.Mp, I, p.P, nullptr, 0, heavy, aph, rsh, stream, bk.start, bk.stop);
    if (st != W4A16_OK) return st;
    MfmaArgs md = ma;
    md.ap = aph;
    md.rs = rsh;
    md.Mp = p.Mp;  // pieces of h: one row per position
    md.arow = nullptr;
    md.K = I;
    md.G = I / kGroup;
    md.qw0 = d.qw0;
    md.sc0 = d.sc0;
    md.qw1 = nullptr;
    md.sc1 = nullptr;
    md.expert_stride = d.expert_stride;
    md.gshift = d.gshift;
    md.N = H;
    md.tiles = (H + kMfmaCols - 1) / kMfmaCols;
    md.gps = md.G;
    md.mode = 0;
    md.out = o;
    md.out_bf16 = xt == W4A16_BF16;
    md.h = nullptr;
    md.extra_plus1 = d.extra_plus1;
    md.qw0x = d.qw0x;
    md.sc0x = d.sc0x;
    md.qw1x = nullptr;
    md.sc1x = nullptr;
    bk = ev.bracket();
    st = launch_mfma(md, p.P, p.max_mitems * md.tiles, stream, bk.start, bk.stop);
    if (st != W4A16_OK) return st;
  }

  // 4. weighted combine in slot order
  bk = ev.bracket();
  const size_t total = static_cast<size_t>(M) * (H / 4);
  const dim3 cgrid(static_cast<unsigned>((total + 255) / 256));
  if (xt == W4A16_BF16)
    hipExtLaunchKernelGGL(combine_kernel<uint16_t>, cgrid, dim3(256), 0, stream, bk.start, bk.stop, 0,
                          reinterpret_cast<const uint16_t*>(o), inv, topk_w, M, top_k, H, shared ? R : -1, y);
  else
    hipExtLaunchKernelGGL(combine_kernel<float>, cgrid, dim3(256), 0, stream, bk.start, bk.stop, 0, o, inv, topk_w,
                          M, top_k, H, shared ? R : -1, y);
  return launch_status();
}
}  // namespace w4

extern "C" w4a16_status_t w4a16_moe_grouped(const void* x, w4a16_dtype_t xt, int32_t M,
                                            const int32_t* topk_ids, const float* topk_w,
                                            int32_t top_k, const w4a16_weight_t* gate,
                                            const w4a16_weight_t* up, const w4a16_weight_t* down,
                                            float* y, void* ws, size_t ws_bytes,
                                            hipStream_t stream) {
  EventMarks none;
  return moe_impl(x, xt, M, topk_ids, topk_w, top_k, gate, up, down, nullptr, nullptr, nullptr, y, ws,
                  ws_bytes, stream, none);
}

extern "C" w4a16_status_t w4a16_moe_grouped_shared(
    const void* x, w4a16_dtype_t xt, int32_t M, const int32_t* topk_ids, const float* topk_w,
    int32_t top_k, const w4a16_weight_t* gate, const w4a16_weight_t* up, const w4a16_weight_t* down,
    const w4a16_weight_t* shared_gate, const w4a16_weight_t* shared_up, const w4a16_weight_t* shared_down,
    float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (shared_gate == nullptr || shared_up == nullptr || shared_down == nullptr) return W4A16_ERR_INVALID_ARG;
  EventMarks none;
  return moe_impl(x, xt, M, topk_ids, topk_w, top_k, gate, up, down, shared_gate, shared_up, shared_down, y,
                  ws, ws_bytes, stream, none);
}

extern "C" w4a16_status_t w4a16_moe_grouped_timed(
    const void* x, w4a16_dtype_t xt, int32_t M, const int32_t* topk_ids, const float* topk_w,
    int32_t top_k, const w4a16_weight_t* gate, const w4a16_weight_t* up,
    const w4a16_weight_t* down, float* y, void* ws, size_t ws_bytes, hipStream_t stream,
    hipEvent_t* events, int32_t capacity, int32_t* recorded) {
  if (capacity < 0 || (capacity > 0 && events == nullptr)) return W4A16_ERR_INVALID_ARG;
  EventMarks ev;
  ev.events = events;
  ev.capacity = capacity;
  w4a16_status_t st = moe_impl(x, xt, M, topk_ids, topk_w, top_k, gate, up, down, nullptr, nullptr, nullptr,
                                y, ws, ws_bytes, stream, ev);
  if (recorded != nullptr) *recorded = ev.recorded;
  return st;
}
