// Top-k selection and renormalised softmax of one token's router logits (one wave).
#pragma once

#include "device.hpp"

namespace moe4 {

// A logit and its expert index as one 64-bit key whose unsigned order is the
// selection order: larger logit first, equal logits -> lower expert index first.
// Bits 39..8 hold the float's order-preserving image, bits 7..0 hold 255 - e (E <= 256).
// NaN counts as -inf and -0 as +0 (they compare equal as floats). Key 0 means "none":
// every real key is larger, since the image of -inf is 0x007fffff.
__device__ __forceinline__ uint64_t topk_key(float l, int e) {
  if (l != l) l = -INFINITY;
  l = l + 0.0f;  // -0 -> +0
  const uint32_t b = __float_as_uint(l);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 8) | (uint64_t)(255 - e);
}
__device__ __forceinline__ int topk_key_index(uint64_t key) { return 255 - (int)(key & 0xffu); }
__device__ __forceinline__ float topk_key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 8);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, kCtrl, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), kCtrl, 0xf, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum of a 64-bit key, returned wave-uniform. Within each row of 16
// lanes: DPP exchanges with lane^1, lane^2 (quad permutes), the mirror lane in the
// half row and the mirror lane in the row; then the four row maxima are combined.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xb1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4e>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
  return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)),
                 max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
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
// (expert index and weight). k rounds of a wave-wide maximum over the keys not yet
// picked; the owner of the maximum drops it. Weights: exp(L_j - L_max) over the sum
// of the selected, i.e. the softmax over all experts renormalised to the selected.
__device__ __forceinline__ void topk_softmax_row(const float* __restrict__ row, int E, int k, int& out_idx,
                                                 float& out_w) {
  const int lane = threadIdx.x & 63;
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? topk_key(row[e], e) : 0ull;
  }
  uint64_t mine = 0;
  for (int s = 0; s < k; ++s) {
    const uint64_t own = max_u64(max_u64(key[0], key[1]), max_u64(key[2], key[3]));
    const uint64_t best = wave_max_u64(own);
#pragma unroll
    for (int j = 0; j < 4; ++j) key[j] = key[j] == best ? 0ull : key[j];
    if (lane == s) mine = best;
  }
  const float lmax = topk_key_value(readlane_u64(mine, 0));
  const float ex = lane < k ? expf(topk_key_value(mine) - lmax) : 0.f;
  out_idx = topk_key_index(mine);
  out_w = ex / wave_sum_fixed(ex);
}

}  // namespace moe4
