// Router logits and top-k softmax.
//
// The TensorFold issue #627 (BobClawblaw's comment of Oct 14) found that a router that
// serialises a row's expert dot products on one multiprocessor was about 6x slower
// than a tiled router that spreads them over many blocks, and that the tiled form
// with a fixed summation order keeps its outputs byte-identical run to run. Both
// properties are kept here: one wave per (expert, token tile), so a decode row's
// experts spread over E waves, and every sum runs in a fixed order.
#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

constexpr int kRouterTokens = 8;  // tokens per wave

// grid (ceil(E/4), ceil(T/8)), block 256: wave w -> expert blockIdx.x*4 + w.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            float* __restrict__ logits, int T, int H,
                                                            int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * kRouterTokens;
  if (e >= E) return;
  const int nt = min(kRouterTokens, T - t0);
  float acc[kRouterTokens];
#pragma unroll
  for (int r = 0; r < kRouterTokens; ++r) acc[r] = 0.f;
  const uint4* wrow = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
  const int nchunk = H >> 3;  // 8 BF16 per 16-byte chunk
  for (int c = lane; c < nchunk; c += kWave) {
    const uint4 wv = wrow[c];
    const float w0 = bf16_lo(wv.x), w1 = bf16_hi(wv.x), w2 = bf16_lo(wv.y), w3 = bf16_hi(wv.y);
    const float w4 = bf16_lo(wv.z), w5 = bf16_hi(wv.z), w6 = bf16_lo(wv.w), w7 = bf16_hi(wv.w);
#pragma unroll
    for (int r = 0; r < kRouterTokens; ++r) {
      if (r < nt) {
        const uint4 xv = reinterpret_cast<const uint4*>(x + (size_t)(t0 + r) * H)[c];
        float a = acc[r];
        a = fmaf(bf16_lo(xv.x), w0, a);
        a = fmaf(bf16_hi(xv.x), w1, a);
        a = fmaf(bf16_lo(xv.y), w2, a);
        a = fmaf(bf16_hi(xv.y), w3, a);
        a = fmaf(bf16_lo(xv.z), w4, a);
        a = fmaf(bf16_hi(xv.z), w5, a);
        a = fmaf(bf16_lo(xv.w), w6, a);
        a = fmaf(bf16_hi(xv.w), w7, a);
        acc[r] = a;
      }
    }
  }
  // Butterfly sum: every lane ends with the same bits (a+b == b+a).
#pragma unroll
  for (int r = 0; r < kRouterTokens; ++r) {
    float v = acc[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && r < nt) logits[(size_t)(t0 + r) * E + e] = v;
  }
}

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// One wave per token (block 256 = 4 tokens). Each lane holds experts lane + 64*j.
// k rounds of a wave-wide arg-max; ties go to the lower expert index; NaN counts as
// -inf so every selected index is in range.
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ w, int T, int E,
                                                           int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
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
      if (valid[j] && better(v[j], lane + 64 * j, bv, bi)) { bv = v[j]; bi = lane + 64 * j; }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == bi) valid[j] = false;
    if (lane == s) { my_val = bv; my_idx = bi; }
  }
  // weights: exp(L_j - L_max) / sum over the selected; L_max is the first pick.
  const float lmax = __shfl(my_val, 0);
  const float ex = lane < k ? expf(my_val - lmax) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_idx;
    w[(size_t)t * k + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H,
                                int E, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((E + 3) / 4, (T + kRouterTokens - 1) / kRouterTokens);
  hipLaunchKernelGGL(router_logits_kernel, grid, dim3(256), 0, s, x, wr, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, int32_t* idx, float* w, int T, int E, int k,
                               hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_softmax_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, idx, w, T, E,
                     k);
  return hipGetLastError();
}

}  // namespace moe4
