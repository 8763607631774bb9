// add_moe_norm: weighted sum of a token's expert outputs, plus the shared expert and
// the residual, then RMSNorm (TensorFold issue #627: the add_moe_norm kernel in the
// table "Median time per launch" and in the Oct 14 per-step breakdown).
//
// One workgroup per token. Each thread keeps its columns' FP32 sum o in registers, so
// o is read and written once; the register arrays are sized per launch to the row
// width and k (instantiations of 1, 2, 4, 8 chunks of 8 columns per thread and 4, 8,
// 16 rows), which sets the occupancy and so the rows in flight. The sum of squares is
// reduced in a fixed order (wave butterfly, then waves 0..3), so outputs are
// bit-identical run to run.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;  // workgroup form: H <= 8 * 8 * 256 = 16384
constexpr int kMaxK = 16;

template <int kC, int kK>
__global__ __launch_bounds__(kThreads) void combine_norm_kernel(
    const uint16_t* __restrict__ y, const int32_t* __restrict__ inv, const float* __restrict__ w,
    const uint16_t* __restrict__ shared_y, const uint16_t* residual, const uint16_t* __restrict__ gamma,
    uint16_t* res_out, uint16_t* __restrict__ norm_out, int H, int k, float eps) {
  __shared__ float wsum[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nchunk = H >> 3;

  float wj[kK];
  int rj[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) {
    wj[j] = j < k ? w[(size_t)t * k + j] : 0.f;
    rj[j] = j < k ? inv[(size_t)t * k + j] : 0;
  }

  // independent loads first (residual, gamma, shared), then the gathered y rows
  float o[kC][8];
  uint4 gv[kC];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int ci = tid + c * kThreads;
    if (ci < nchunk) {
      const uint4 rv = reinterpret_cast<const uint4*>(residual + (size_t)t * H)[ci];
      gv[c] = reinterpret_cast<const uint4*>(gamma)[ci];
      const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[c][2 * q] = bf16_lo(rw[q]);
        o[c][2 * q + 1] = bf16_hi(rw[q]);
      }
      uint4 yv[kK];
#pragma unroll
      for (int j = 0; j < kK; ++j)
        if (j < k) yv[j] = reinterpret_cast<const uint4*>(y + (size_t)rj[j] * H)[ci];
#pragma unroll
      for (int j = 0; j < kK; ++j) {
        if (j < k) {
          const uint32_t yw[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[c][2 * q] = fmaf(wj[j], bf16_lo(yw[q]), o[c][2 * q]);
            o[c][2 * q + 1] = fmaf(wj[j], bf16_hi(yw[q]), o[c][2 * q + 1]);
          }
        }
      }
      if (shared_y) {
        const uint4 sv = reinterpret_cast<const uint4*>(shared_y + (size_t)t * H)[ci];
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[c][2 * q] += bf16_lo(sw[q]);
          o[c][2 * q + 1] += bf16_hi(sw[q]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(o[c][e], o[c][e], ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  const float total = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float scale = 1.0f / sqrtf(total / (float)H + eps);

#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int ci = tid + c * kThreads;
    if (ci < nchunk) {
      const uint32_t gw[4] = {gv[c].x, gv[c].y, gv[c].z, gv[c].w};
      uint4 ov, nv;
      uint32_t* op = &ov.x;
      uint32_t* np = &nv.x;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        op[q] = pack_bf16x2(o[c][2 * q], o[c][2 * q + 1]);
        np[q] = pack_bf16x2(o[c][2 * q] * scale * bf16_lo(gw[q]), o[c][2 * q + 1] * scale * bf16_hi(gw[q]));
      }
      reinterpret_cast<uint4*>(res_out + (size_t)t * H)[ci] = ov;
      reinterpret_cast<uint4*>(norm_out + (size_t)t * H)[ci] = nv;
    }
  }
}

}  // namespace

hipError_t launch_combine_norm(const uint16_t* y, const int32_t* inv, const float* w,
                               const uint16_t* shared_y, const uint16_t* residual,
                               const uint16_t* gamma, uint16_t* res_out, uint16_t* norm_out, int T,
                               int H, int k, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // the smallest register arrays that hold a thread's chunks and a token's k rows (the
  // registers set the occupancy, and with it how many rows are in flight)
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(T), dim3(kThreads), 0, s, y, inv, w, shared_y, residual, gamma, res_out,
                       norm_out, H, k, eps);
    return hipGetLastError();
  };
  auto by_k = [&](auto C) {
    constexpr int c = decltype(C)::value;
    if (k <= 4) return go(combine_norm_kernel<c, 4>);
    if (k <= 8) return go(combine_norm_kernel<c, 8>);
    return go(combine_norm_kernel<c, kMaxK>);
  };
  const int nc = (H / 8 + kThreads - 1) / kThreads;  // chunks per thread
  if (nc <= 1) return by_k(std::integral_constant<int, 1>{});
  if (nc <= 2) return by_k(std::integral_constant<int, 2>{});
  if (nc <= 4) return by_k(std::integral_constant<int, 4>{});
  return by_k(std::integral_constant<int, kMaxChunks>{});
}

}  // namespace moe4
