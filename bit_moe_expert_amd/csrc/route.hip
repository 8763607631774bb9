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
#include "topk.hpp"

namespace moe4 {

namespace {

constexpr int kRouterTokens = 8;  // tokens per workgroup

// grid (E, ceil(T/8)), block 256: one workgroup per expert and token group; the four
// waves split H, each lane takes a contiguous 8-element chunk per 512 columns, so a
// lane issues all its loads at once. Partials are summed by a wave butterfly and
// then across the waves in order through LDS.
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            float* __restrict__ logits, int T, int H,
                                                            int E) {
  __shared__ float part[4][kRouterTokens];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterTokens;
  const int nt = min(kRouterTokens, T - t0);
  float acc[kRouterTokens];
#pragma unroll
  for (int r = 0; r < kRouterTokens; ++r) acc[r] = 0.f;
  const uint4* wrow = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
  const int nchunk = H >> 3;  // 8 BF16 per 16-byte chunk
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    const uint4 wv = wrow[c];
    uint4 xv[kRouterTokens];
#pragma unroll
    for (int r = 0; r < kRouterTokens; ++r)
      xv[r] = r < nt ? reinterpret_cast<const uint4*>(x + (size_t)(t0 + r) * H)[c] : make_uint4(0, 0, 0, 0);
    const float w0 = bf16_lo(wv.x), w1 = bf16_hi(wv.x), w2 = bf16_lo(wv.y), w3 = bf16_hi(wv.y);
    const float w4 = bf16_lo(wv.z), w5 = bf16_hi(wv.z), w6 = bf16_lo(wv.w), w7 = bf16_hi(wv.w);
#pragma unroll
    for (int r = 0; r < kRouterTokens; ++r) {
      float a = acc[r];
      a = fmaf(bf16_lo(xv[r].x), w0, a);
      a = fmaf(bf16_hi(xv[r].x), w1, a);
      a = fmaf(bf16_lo(xv[r].y), w2, a);
      a = fmaf(bf16_hi(xv[r].y), w3, a);
      a = fmaf(bf16_lo(xv[r].z), w4, a);
      a = fmaf(bf16_hi(xv[r].z), w5, a);
      a = fmaf(bf16_lo(xv[r].w), w6, a);
      a = fmaf(bf16_hi(xv[r].w), w7, a);
      acc[r] = a;
    }
  }
  // Butterfly sum: every lane ends with the same bits (a+b == b+a).
#pragma unroll
  for (int r = 0; r < kRouterTokens; ++r) {
    float v = acc[r];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) part[wave][r] = v;
  }
  __syncthreads();
  if (threadIdx.x < nt) {
    const int r = threadIdx.x;
    logits[(size_t)(t0 + r) * E + e] = ((part[0][r] + part[1][r]) + part[2][r]) + part[3][r];
  }
}



// One wave per token (block 256 = 4 tokens).
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ w, int T, int E,
                                                           int k) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int oi;
  float ow;
  topk_softmax_row(logits + (size_t)t * E, E, k, oi, ow);
  const int lane = threadIdx.x & 63;
  if (lane < k) {
    idx[(size_t)t * k + lane] = oi;
    w[(size_t)t * k + lane] = ow;
  }
}

}  // namespace

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H,
                                int E, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid(E, (T + kRouterTokens - 1) / kRouterTokens);
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
