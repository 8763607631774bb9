// Top-k selection and renormalised softmax of one token's router logits (one wave).
#pragma once

#include "device.hpp"

namespace moe4 {

// A logit's order-preserving 32-bit image: unsigned order of images = float order of
// logits, NaN counting as -inf and -0 as +0 (they compare equal as floats). Image 0 is
// below every real one (the image of -inf is 0x007fffff) and marks a picked expert.
__device__ __forceinline__ uint32_t topk_image(float l) {
  if (l != l) l = -INFINITY;
  l = l + 0.0f;  // -0 -> +0
  const uint32_t b = __float_as_uint(l);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float topk_image_value(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

// Wave-wide maximum of a 32-bit value, returned wave-uniform. Within each row of 16
// lanes: DPP exchanges with lane^1, lane^2 (quad permutes), the mirror lane in the
// half row and the mirror lane in the row; then the four row maxima are combined.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));  // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Wave-wide sum with a fixed combination order (the same bits on every lane and run).
__device__ __forceinline__ float wave_sum_fixed(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Top-k of one token's logits by the calling wave; lane j < k returns the j-th pick
// (expert index and weight). Lane l holds experts l, l + 64, l + 128, l + 192 as
// images. k rounds: the wave-wide maximum image, then the lowest expert index holding
// it (ballots per expert group, lowest group first, then lowest lane), which is
// dropped. So the order is larger logit first, equal logits -> lower expert index.
// Weights: exp(L_j - L_max) over the sum of the selected, i.e. the softmax over all
// experts renormalised to the selected.
__device__ __forceinline__ void topk_softmax_row(const float* __restrict__ row, int E, int k, int& out_idx,
                                                 float& out_w) {
  const int lane = threadIdx.x & 63;
  uint32_t img[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    img[j] = e < E ? topk_image(row[e]) : 0u;
  }
  int mine_idx = 0;
  uint32_t mine = 0;
  for (int s = 0; s < k; ++s) {
    const uint32_t best = wave_max_u32(max(max(img[0], img[1]), max(img[2], img[3])));
    int pick = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t b = __ballot(img[j] == best);
      if (pick < 0 && b) pick = 64 * j + (__ffsll((long long)b) - 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) img[j] = lane + 64 * j == pick ? 0u : img[j];
    if (lane == s) {
      mine_idx = pick;
      mine = best;
    }
  }
  const float lmax = topk_image_value(__builtin_amdgcn_readlane((int)mine, 0));
  const float ex = lane < k ? expf(topk_image_value(mine) - lmax) : 0.f;
  out_idx = mine_idx;
  out_w = ex / wave_sum_fixed(ex);
}

}  // namespace moe4
