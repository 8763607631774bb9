// Block-scaled FP8 activations for the W4A8 prefill variant: each block of 32
// consecutive BF16 values along a row gets a power-of-two scale 2^e (stored as an
// E8M0 byte, e + 127), e the smallest integer for which the block's largest magnitude
// times 2^-e is at most 448, the largest OCP E4M3 value (so nothing saturates; e = 0
// for an all-zero block; e clamped to [-127, 127]), and every value times 2^-e is
// rounded to E4M3, nearest with ties to even. The FP8 prompt-matmul option of the
// Qiita TensorFold 1.1.x article ("Why it still does not reach 0.6.6") and the PR804
// article's NVFP4 section (W4A16 against lower-precision activations) are the
// sources; the block size and the scale format are those the gfx950 block-scaled
// MFMA consumes (one E8M0 scale per 32 K values of a row).
//
// The scale decision and the rounding are exact integer decisions on exact values
// (the scaling is by a power of two), so any correct implementation gives the same
// bytes.
#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

constexpr int kBlock = 32;

// One thread per block of 32 values: 4 x 16-byte loads, one 32-byte store of codes
// and one scale byte.
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const uint16_t* __restrict__ x, long long nblocks,
                                                          uint8_t* __restrict__ q, uint8_t* __restrict__ e_out) {
  const long long b = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + b * kBlock);
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[i];
  u32x4 out[2];
  const int e = mxfp8_block(v, out);
  u32x4* dst = reinterpret_cast<u32x4*>(q + b * kBlock);
  dst[0] = out[0];
  dst[1] = out[1];
  e_out[b] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_mxfp8_quant(const uint16_t* x, long long rows, int K, uint8_t* q, uint8_t* e, hipStream_t s) {
  const long long nblocks = rows * (K / kBlock);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s, x, nblocks, q, e);
  return hipGetLastError();
}

}  // namespace moe4
