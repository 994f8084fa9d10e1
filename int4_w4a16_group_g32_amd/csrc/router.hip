// Router: top-k experts per token and their gate weights.
//
// Web page "The Final Wire: How a Single Edit Integrated INT4 Quantization into
// a Native DDTree Inference Engine", section "What the Edit Actually Changes":
// for each token the router selects top-k experts.  The pages give no gating
// rule; this library takes the k largest logits in descending order (equal
// logits in ascending expert index) and softmax over those k logits as the
// gate weights.
#include <cfloat>
#include <climits>

#include "common.h"

namespace w4 {
namespace {

constexpr int kTopkThreads = 256;                 // four token rows per workgroup
constexpr int kTopkPerLane = 16;                  // experts per lane: E <= 1024
constexpr int kTopkMaxE = kWave * kTopkPerLane;
constexpr int kTopkMaxK = 32;

// (value, index) order of the selection: larger value first, then smaller index.
__device__ __forceinline__ bool before(float va, int ea, float vb, int eb) {
  return va > vb || (va == vb && ea < eb);
}

// One wave per token row.  Lane l holds the logits of experts l, l + 64, ...;
// each of the k rounds takes the lane's best untaken expert, reduces (value,
// index) across the wave with butterfly shuffles, marks the winner taken on
// its lane and parks it on lane `round`.  The weights are then a softmax over
// lanes 0 .. k-1: exponentials relative to the first (largest) logit, their
// sum reduced onto lane 0 and broadcast, one division each.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ logits, int M, int E,
                                                            int k, int32_t* __restrict__ ids,
                                                            float* __restrict__ w) {
  const int row = static_cast<int>(blockIdx.x) * (kTopkThreads / kWave) + wave_id();
  if (row >= M) return;
  const int lane = lane_id();
  const float* lr = logits + static_cast<size_t>(row) * E;
  float v[kTopkPerLane];
#pragma unroll
  for (int j = 0; j < kTopkPerLane; ++j) {
    const int e = lane + kWave * j;
    v[j] = e < E ? lr[e] : -FLT_MAX;
  }
  uint32_t taken = 0;  // bit j: expert lane + 64j is chosen (or absent)
#pragma unroll
  for (int j = 0; j < kTopkPerLane; ++j)
    if (lane + kWave * j >= E) taken |= 1u << j;

  float mine_v = 0.0f;
  int mine_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -FLT_MAX;
    int be = INT_MAX;
#pragma unroll
    for (int j = 0; j < kTopkPerLane; ++j) {
      const int e = lane + kWave * j;
      if (!((taken >> j) & 1u) && before(v[j], e, bv, be)) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    if (lane == r) {
      mine_v = bv;
      mine_e = be;
    }
  }
  const float vmax = __shfl(mine_v, 0);
  const float z = lane < k ? expf(mine_v - vmax) : 0.0f;
  float sum = z;
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) sum += __shfl_down(sum, off);
  sum = __shfl(sum, 0);
  if (lane < k) {
    ids[static_cast<size_t>(row) * k + lane] = mine_e;
    w[static_cast<size_t>(row) * k + lane] = z / sum;
  }
}

}  // namespace
}  // namespace w4

extern "C" w4a16_status_t w4a16_moe_topk(const float* logits, int32_t M, int32_t E, int32_t top_k,
                                         int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  using namespace w4;
  if (M < 0 || E < 1 || top_k < 1 || top_k > E) return W4A16_ERR_INVALID_ARG;
  if (E > kTopkMaxE || top_k > kTopkMaxK) return W4A16_ERR_UNSUPPORTED;
  if (M == 0) return W4A16_OK;
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr) return W4A16_ERR_INVALID_ARG;
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w)) return W4A16_ERR_INVALID_ARG;
  const int rows_per_wg = kTopkThreads / kWave;
  const unsigned grid = static_cast<unsigned>((M + rows_per_wg - 1) / rows_per_wg);
  topk_kernel<<<grid, kTopkThreads, 0, stream>>>(logits, M, E, top_k, topk_ids, topk_w);
  return launch_status();
}
