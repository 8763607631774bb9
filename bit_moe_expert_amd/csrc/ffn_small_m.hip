// Grouped W4A16 expert FFN for few rows per expert (decode and batched decode).
//
// Decode is bound by reading the touched experts' weights once (the bandwidth-budget
// article on GB10, section "Mechanism: decode is bandwidth-bound, prefill is
// compute-bound"), and batching raises throughput by sharing each weight read across
// the rows of the batch (same article, "Batching changes the arithmetic"). So each
// weight byte is read from HBM once per call and used for every row its expert got.
//
// Work split. Grid (N-tile, expert); empty experts exit at once. A workgroup (4
// waves) owns 64 weight rows (up: 32 gate + the matching 32 up rows, so SwiGLU can
// be applied in the epilogue; down: 64 rows of W2) and splits K into 128-wide steps
// dealt round-robin to its waves; the four partial sums are added in a fixed order
// through LDS at the end.
//
// Per step a lane streams 16 bytes (32 codes) of one weight row plus the row's two
// E4M3 block scales, dequantises them exactly into BF16 (code * scale has at most 6
// significant bits) and feeds four 16x16x32 BF16 MFMAs per 16-row tile of the
// expert's rows. Up to two row tiles (32 rows) share one pass over the weights;
// more rows take further passes (correct for any count, fast for few).
#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

constexpr int kKStep = 128;   // K per step: 4 lane groups x 32 codes
constexpr int kBlocks = 4;    // 16-row weight blocks per workgroup
constexpr int kMaxTiles = 2;  // 16-row activation tiles per pass

struct SmallMArgs {
  const uint16_t* act;       // up: x [T][H]; down: h [R][I]
  const int32_t* offsets;    // [G+1] or NULL (dense: one group of T rows)
  const int32_t* perm_src;   // up only: row -> flat pair (token = pair / k); NULL = identity
  int k;
  int T;
  const uint8_t* packed;     // [G][N][K/2]
  const uint8_t* scales;     // [G][N][K/16]
  const float* tscale;       // [G]
  int N, K, I;               // up: N = 2I, K = H; down: N = H, K = I
  uint16_t* out;             // up: h [R][I]; down: y [R][N]
};

template <bool kUp, int kTiles>
__device__ __forceinline__ void small_m_pass(const SmallMArgs& a, int g, int r0, int M, int pass_base,
                                             float4* red /* LDS [4][kBlocks][64] */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rn = lane & 15;  // weight row within a block; activation row within a tile
  const int kq = lane >> 4;  // lane group: which 32 codes of the 128-wide step
  const int K = a.K;
  const size_t row_bytes = (size_t)K / 2, row_scales = (size_t)K / 16;
  const uint8_t* wp = a.packed + (size_t)g * a.N * row_bytes;
  const uint8_t* sp = a.scales + (size_t)g * a.N * row_scales;

  // the four weight rows this lane streams (one per block)
  size_t wrow[kBlocks], srow[kBlocks];
#pragma unroll
  for (int b = 0; b < kBlocks; ++b) {
    int n;
    if (kUp) n = (b < 2 ? 0 : a.I) + blockIdx.x * 32 + (b & 1) * 16 + rn;
    else n = blockIdx.x * 64 + b * 16 + rn;
    wrow[b] = (size_t)n * row_bytes;
    srow[b] = (size_t)n * row_scales;
  }
  // activation rows of this lane in each tile
  const uint16_t* arow[kTiles];
  bool aval[kTiles];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int m = pass_base + t * 16 + rn;
    aval[t] = m < M;
    const int r = r0 + (aval[t] ? m : 0);
    int src = r;
    if (kUp) src = a.perm_src ? a.perm_src[r] / a.k : r;
    arow[t] = a.act + (size_t)src * K;
  }

  f32x4 acc[kTiles][kBlocks];
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K / kKStep;
  for (int it = wave; it < nsteps; it += 4) {
    const int kb = it * kKStep + kq * 32;
    u32x4 wq[kBlocks];
    uint32_t sc[kBlocks];
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      wq[b] = *reinterpret_cast<const u32x4*>(wp + wrow[b] + kb / 2);
      sc[b] = *reinterpret_cast<const uint16_t*>(sp + srow[b] + kb / 16);
    }
    float s0[kBlocks], s1[kBlocks];
#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
      s0[b] = e4m3_to_f32<0>(sc[b]);
      s1[b] = e4m3_to_f32<1>(sc[b]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 av[kTiles];
#pragma unroll
      for (int t = 0; t < kTiles; ++t)
        av[t] = aval[t] ? *reinterpret_cast<const u32x4*>(arow[t] + kb + 8 * j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < kBlocks; ++b) {
        const u32x4 bw = dequant8(wq[b][j], j < 2 ? s0[b] : s1[b]);
#pragma unroll
        for (int t = 0; t < kTiles; ++t) acc[t][b] = mfma16x16x32(av[t], bw, acc[t][b]);
      }
    }
  }

  // Cross-wave sum (waves 0..3 in order), then the epilogue, one tile at a time.
  const float ts = a.tscale[g];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    __syncthreads();
#pragma unroll
    for (int b = 0; b < kBlocks; ++b)
      red[(wave * kBlocks + b) * 64 + lane] = make_float4(acc[t][b][0], acc[t][b][1], acc[t][b][2], acc[t][b][3]);
    __syncthreads();
    const int mbase = pass_base + t * 16 + 4 * kq;  // rows mbase..mbase+3, column rn
    if (kUp) {
      if (wave < 2) {
        float4 gs = red[(0 * kBlocks + wave) * 64 + lane];
        float4 us = red[(0 * kBlocks + wave + 2) * 64 + lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float4 gg = red[(w * kBlocks + wave) * 64 + lane];
          const float4 uu = red[(w * kBlocks + wave + 2) * 64 + lane];
          gs.x += gg.x; gs.y += gg.y; gs.z += gg.z; gs.w += gg.w;
          us.x += uu.x; us.y += uu.y; us.z += uu.z; us.w += uu.w;
        }
        const float gv[4] = {gs.x, gs.y, gs.z, gs.w}, uv[4] = {us.x, us.y, us.z, us.w};
        const int col = blockIdx.x * 32 + wave * 16 + rn;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mbase + r < M)
            a.out[(size_t)(r0 + mbase + r) * a.I + col] = f32_to_bf16(silu_mul(ts * gv[r], ts * uv[r]));
      }
    } else {
      float4 ds = red[(0 * kBlocks + wave) * 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float4 dd = red[(w * kBlocks + wave) * 64 + lane];
        ds.x += dd.x; ds.y += dd.y; ds.z += dd.z; ds.w += dd.w;
      }
      const float dv[4] = {ds.x, ds.y, ds.z, ds.w};
      const int col = blockIdx.x * 64 + wave * 16 + rn;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (mbase + r < M) a.out[(size_t)(r0 + mbase + r) * a.N + col] = f32_to_bf16(ts * dv[r]);
    }
  }
}

template <bool kUp>
__global__ __launch_bounds__(256) void ffn_small_m_kernel(SmallMArgs a) {
  __shared__ float4 red[4 * kBlocks * 64];
  const int g = blockIdx.y;
  int r0 = 0, M = a.T;
  if (a.offsets) {
    r0 = a.offsets[g];
    M = a.offsets[g + 1] - r0;
  }
  if (M <= 0) return;
  for (int pass_base = 0; pass_base < M; pass_base += 16 * kMaxTiles) {
    const int tiles = min(kMaxTiles, (M - pass_base + 15) / 16);
    switch (tiles) {
      case 1: small_m_pass<kUp, 1>(a, g, r0, M, pass_base, red); break;
      default: small_m_pass<kUp, 2>(a, g, r0, M, pass_base, red); break;
    }
  }
}

}  // namespace

hipError_t launch_ffn_up(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                         int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  SmallMArgs a{x, offsets, perm_src, k, T, w13.packed, w13.scales, w13.tscale, 2 * I, H, I, h};
  hipLaunchKernelGGL(ffn_small_m_kernel<true>, dim3(I / 32, G), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ffn_down(const uint16_t* h, const int32_t* offsets, int T, int G, int H, int I,
                           W4View w2, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  SmallMArgs a{h, offsets, nullptr, 1, T, w2.packed, w2.scales, w2.tscale, H, I, I, y};
  hipLaunchKernelGGL(ffn_small_m_kernel<false>, dim3(H / 64, G), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe4
