// add_rmsnorm and group_rmsnorm: the two RMSNorm glue kernels that run beside the MoE
// layer in a decode step (TensorFold issue #627: add_rmsnorm in the Oct 10 list of the
// other glue ops, add_rmsnorm and group_rmsnorm in the Oct 14 per-step breakdown of
// launches).
//
//   add_rmsnorm:   o = x + residual, n = o / sqrt(mean(o^2) + eps) * gamma over the row;
//   group_rmsnorm: n = x / sqrt(mean_group(x^2) + eps) * gamma, each contiguous group of
//                  `group` columns of a row normalised by its own mean square.
//
// One workgroup of 256 threads per row. Each thread keeps its 16-byte chunks (8
// columns) of the FP32 row in registers, so every input is read once and every output
// written once; the LDS holds one FP32 per chunk and per group. (Blocks of 64 or 128
// threads per row measured the same or slower.) The sums of squares are reduced in a
// fixed order (per chunk, then per group: by one wave for groups of 64 chunks or more,
// a strided serial sum per lane and a butterfly, else by one thread in chunk order), so
// outputs are bit-identical from run to run and do not depend on T. Sums are FP32:
// values whose squares overflow FP32 are out of range. Every thread reads all of its
// chunks before the barrier and writes only those chunks after it, so outputs may alias
// inputs.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;                   // chunks per thread: H <= 8 * 8 * 256
constexpr int kMaxCols = kMaxChunks * kThreads * 8;

template <int kC>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const uint16_t* x, const uint16_t* residual,
                                                           const uint16_t* __restrict__ gamma,
                                                           uint16_t* res_out, uint16_t* norm_out, int H,
                                                           int group, float eps) {
  extern __shared__ float smem[];
  float* part = smem;                 // [H / 8]: sum of squares of each chunk
  float* gscale = smem + (H >> 3);    // [H / group]: 1 / rms of each group
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = H >> 3, cg = group >> 3, ngroup = H / group;

  float o[kC][8];
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int ci = tid + c * kThreads;
    if (ci < nchunk) {
      const uint4 xv = reinterpret_cast<const uint4*>(x + (size_t)t * H)[ci];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[c][2 * q] = bf16_lo(xw[q]);
        o[c][2 * q + 1] = bf16_hi(xw[q]);
      }
      if (residual) {
        const uint4 rv = reinterpret_cast<const uint4*>(residual + (size_t)t * H)[ci];
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[c][2 * q] += bf16_lo(rw[q]);
          o[c][2 * q + 1] += bf16_hi(rw[q]);
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(o[c][e], o[c][e], ss);
      part[ci] = ss;
    }
  }
  __syncthreads();
  if (cg >= kWave) {
    // wide groups: group g is reduced by wave g % (waves); lane l sums chunks l, l + 64, ...
    // of the group in order, then the 64 lane sums are combined by a butterfly
    for (int g = wave; g < ngroup; g += kThreads / kWave) {
      float s = 0.f;
      for (int j = lane; j < cg; j += kWave) s += part[g * cg + j];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) gscale[g] = 1.0f / sqrtf(s / (float)group + eps);
    }
  } else {
    // narrow groups (fewer than 64 chunks): one thread sums a group's chunks in order
    for (int g = tid; g < ngroup; g += kThreads) {
      float s = 0.f;
      for (int j = 0; j < cg; ++j) s += part[g * cg + j];
      gscale[g] = 1.0f / sqrtf(s / (float)group + eps);
    }
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int ci = tid + c * kThreads;
    if (ci < nchunk) {
      const float scale = gscale[ci / cg];
      const uint4 gv = reinterpret_cast<const uint4*>(gamma)[ci];
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
      uint4 ov, nv;
      uint32_t* op = &ov.x;
      uint32_t* np = &nv.x;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        op[q] = pack_bf16x2(o[c][2 * q], o[c][2 * q + 1]);
        np[q] = pack_bf16x2(o[c][2 * q] * scale * bf16_lo(gw[q]), o[c][2 * q + 1] * scale * bf16_hi(gw[q]));
      }
      if (res_out) reinterpret_cast<uint4*>(res_out + (size_t)t * H)[ci] = ov;
      reinterpret_cast<uint4*>(norm_out + (size_t)t * H)[ci] = nv;
    }
  }
}

}  // namespace

bool rmsnorm_shape_ok(int H, int group) {
  return H > 0 && H % 8 == 0 && H <= kMaxCols && group > 0 && group % 8 == 0 && H % group == 0;
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                          uint16_t* res_out, uint16_t* norm_out, int T, int H, int group, float eps,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const size_t lds = (size_t)(H / 8 + H / group) * sizeof(float);
  auto go = [&](auto C) {
    constexpr int c = decltype(C)::value;
    hipLaunchKernelGGL(rmsnorm_kernel<c>, dim3(T), dim3(kThreads), lds, s, x, residual, gamma, res_out,
                       norm_out, H, group, eps);
    return hipGetLastError();
  };
  // the smallest register array that holds a thread's chunks
  const int nc = (H / 8 + kThreads - 1) / kThreads;
  if (nc <= 1) return go(std::integral_constant<int, 1>{});
  if (nc <= 2) return go(std::integral_constant<int, 2>{});
  if (nc <= 4) return go(std::integral_constant<int, 4>{});
  return go(std::integral_constant<int, kMaxChunks>{});
}

}  // namespace moe4
