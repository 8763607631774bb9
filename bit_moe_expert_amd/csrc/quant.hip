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

// FP16 activation rows for the up projection's GEMM form. Row t gets the exponent
// e_t, the smallest integer for which its largest magnitude times 2^-e_t is below 2^15
// (e_t = 0 for a row of zeros; NaN is ignored), and x16[t][k] = x[t][k] * 2^-e_t
// rounded to FP16, nearest with ties to even. A BF16 value has 8 significant bits, so
// the scaled value is exact in FP16 unless it lies below 2^-17, i.e. more than 2^31
// under the row's largest magnitude. One workgroup of 256 threads per row, the row's
// 16-byte chunks held in registers between the maximum and the conversion.
constexpr int kF16Threads = 256;
constexpr int kF16Chunks = 8;  // 16-byte chunks a thread holds: K <= 256 * 8 * 8 = 16384

__global__ __launch_bounds__(kF16Threads) void act_f16_kernel(const uint16_t* __restrict__ x, int K,
                                                              uint16_t* __restrict__ x16,
                                                              int32_t* __restrict__ xexp) {
  __shared__ uint32_t wmax[kF16Threads / 64];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x, cpr = K / 8;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * K);
  u32x4 v[kF16Chunks];
  uint32_t amax = 0;  // BF16 magnitudes (NaN excluded) order as their bit patterns
#pragma unroll
  for (int u = 0; u < kF16Chunks; ++u) {
    const int c = u * kF16Threads + tid;
    if (c < cpr) {
      v[u] = src[c];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = v[u][j] & 0x7fffu, hi = (v[u][j] >> 16) & 0x7fffu;
        amax = max(amax, lo <= 0x7f80u ? lo : 0u);
        amax = max(amax, hi <= 0x7f80u ? hi : 0u);
      }
    }
  }
  // workgroup maximum: across each wave by lane exchanges, then across the 4 waves
  // through LDS
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, d, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  int e = 0;
  if (amax != 0) e = __builtin_amdgcn_frexp_expf(__uint_as_float(amax << 16)) - 1 - 14;
  if (tid == 0) xexp[row] = e;
  uint32_t* dst = reinterpret_cast<uint32_t*>(x16 + row * K);
#pragma unroll
  for (int u = 0; u < kF16Chunks; ++u) {
    const int c = u * kF16Threads + tid;
    if (c < cpr) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 h = {(_Float16)__builtin_ldexpf(bf16_lo(v[u][j]), -e), (_Float16)__builtin_ldexpf(bf16_hi(v[u][j]), -e)};
        o[j] = __builtin_bit_cast(uint32_t, h);
      }
      reinterpret_cast<u32x4*>(dst)[c] = o;
    }
  }
}

}  // namespace

hipError_t launch_act_f16(const uint16_t* x, long long rows, int K, uint16_t* x16, int32_t* xexp, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(act_f16_kernel, dim3((unsigned)rows), dim3(kF16Threads), 0, s, x, K, x16, xexp);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quant(const uint16_t* x, long long rows, int K, uint8_t* q, uint8_t* e, hipStream_t s) {
  const long long nblocks = rows * (K / kBlock);
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s, x, nblocks, q, e);
  return hipGetLastError();
}

}  // namespace moe4
