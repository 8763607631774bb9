// Top-k selection and renormalised softmax of one token's router logits (one wave).
#pragma once

#include "device.hpp"

namespace moe4 {

__device__ __forceinline__ bool topk_better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Top-k of one token's logits by the calling wave; lane j < k returns the j-th pick
// (expert index and weight).
// k rounds of a wave-wide arg-max; ties go to the lower expert index; NaN counts as
// -inf so every selected index is in range. Weights: exp(L_j - L_max) over the sum
// of the selected, i.e. the softmax over all experts renormalised to the selected.
__device__ __forceinline__ void topk_softmax_row(const float* __restrict__ row, int E, int k, int& out_idx,
                                                 float& out_w) {
  const int lane = threadIdx.x & 63;
  float v[4];
  bool valid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < E;
    float l = valid[j] ? row[e] : -INFINITY;
    v[j] = (l != l) ? -INFINITY : l;
  }
  float my_val = 0.f;
  int my_idx = 0;
  for (int s = 0; s < k; ++s) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (valid[j] && topk_better(v[j], lane + 64 * j, bv, bi)) { bv = v[j]; bi = lane + 64 * j; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (topk_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == bi) valid[j] = false;
    if (lane == s) { my_val = bv; my_idx = bi; }
  }
  const float lmax = __shfl(my_val, 0);
  const float ex = lane < k ? expf(my_val - lmax) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  out_idx = my_idx;
  out_w = ex / sum;
}


}  // namespace moe4
