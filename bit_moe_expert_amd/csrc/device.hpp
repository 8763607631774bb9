// Device helpers shared by the libmoe4 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe4 {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// BF16 <-> FP32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Two FP32 -> packed BF16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) { return (uint16_t)(pack_bf16x2(a, 0.f) & 0xffffu); }

// ---------------------------------------------------------------------------
// 4-bit weights
// ---------------------------------------------------------------------------
// E4M3 (OCP) block-scale code in byte `sel` of v -> FP32 (v_cvt_f32_fp8, OCP on gfx950).
template <int sel>
__device__ __forceinline__ float e4m3_to_f32(uint32_t v) { return __builtin_amdgcn_cvt_f32_fp8((int)v, sel); }

// Byte `sel` of `codes` (two E2M1 codes, low nibble first) -> two FP32 values.
// The hardware conversion applies only the exponent of its scale operand, so it is
// called with 1.0 and the E4M3 block scale is multiplied in afterwards; the product
// of a 2-significant-bit code and a 4-significant-bit scale is exact in BF16.
template <int sel>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, sel);
}

// Eight codes (one dword, element 0 in the lowest nibble) times one block scale ->
// eight BF16 weights as 4 dwords, element order preserved (exact).
__device__ __forceinline__ u32x4 dequant8(uint32_t codes, float s) {
  f32x2 a = e2m1x2_to_f32<0>(codes);
  f32x2 b = e2m1x2_to_f32<1>(codes);
  f32x2 c = e2m1x2_to_f32<2>(codes);
  f32x2 d = e2m1x2_to_f32<3>(codes);
  u32x4 r;
  r[0] = pack_bf16x2(a[0] * s, a[1] * s);
  r[1] = pack_bf16x2(b[0] * s, b[1] * s);
  r[2] = pack_bf16x2(c[0] * s, c[1] * s);
  r[3] = pack_bf16x2(d[0] * s, d[1] * s);
  return r;
}

// FP16 form of the same: the two E4M3 scales of a dword's low half -> FP16 (exact:
// E4M3 values lie in FP16's normal range with 4 significant bits), and eight codes
// times one of them -> eight FP16 weights (exact: at most 6 significant bits, between
// 2^-10 and 2688). Two instructions per pair of weights instead of four.
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t v) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false); }
__device__ __forceinline__ u32x4 dequant8_f16(uint32_t codes, _Float16 s) {
  const f16x2 ss = {s, s};
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss);
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss);
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss);
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss);
  return r;
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: shifts within rows of
// 16 lanes (lanes shifted in from before the row read 0), then row 0's total added to
// rows 1 and 3 and rows 0-1's total to rows 2 and 3 (DPP row broadcasts). Every lane
// of the wave must be active. (Lane shuffles, __shfl_up, go through LDS, one round trip
// a step: the prefill GEMM's tile schedule, three scans of four rounds of experts, took
// several microseconds of each workgroup's prologue that way.)
__device__ __forceinline__ int wave_incl_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// ---------------------------------------------------------------------------
// MFMA wrappers (operand layouts checked on gfx950):
//  16x16x32 bf16: lane l supplies A[l%16][kslot(l/16, 0..7)], B[kslot(l/16, 0..7)][l%16];
//                 D[4*(l/16)+r][l%16] = acc[r].
//  32x32x16 bf16: lane l supplies A[l%32][kslot(l/32, 0..7)], B[kslot(l/32, 0..7)][l%32];
//                 D[8*(r/4)+4*(l/32)+r%4][l%32] = acc[r].
// A and B only have to agree on which K each (lane group, slot) stands for.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Buffer-resource loads: a wave-uniform base and byte range, a per-lane 32-bit offset.
// Offsets at or past the range read as zero instead of touching memory.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr int kBufResFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
__device__ __forceinline__ BufRes make_res(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufResFlags);
}
// 16 bytes, streamed past the caches (nt)
__device__ __forceinline__ u32x4 load_b128_nt(BufRes r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ uint32_t load_b16(BufRes r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// Block-scaled FP8 activations (the W4A8 prefill variant): 32 consecutive BF16
// values (4 dwords of pairs, element order low half first) -> 32 OCP E4M3 bytes and
// the block's power-of-two exponent e (stored by callers as the E8M0 byte e + 127).
// e is the smallest integer for which the block's largest magnitude times 2^-e is at
// most 448 (so nothing saturates), 0 for an all-zero block, clamped to [-127, 127];
// each value times 2^-e (exact) is rounded to E4M3, nearest with ties to even
// (v_cvt_pk_fp8_f32; checked bit for bit against that rule on gfx950, including the
// subnormal range).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mxfp8_block(const u32x4 v[4], u32x4 out[2]) {
  uint32_t amax = 0;  // BF16 magnitudes order as their bit patterns
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = max(amax, max(v[i][j] & 0x7fffu, (v[i][j] >> 16) & 0x7fffu));
  int e = 0;
  if (amax != 0) {
    const float a = __uint_as_float(amax << 16);
    const int E = __builtin_amdgcn_frexp_expf(a) - 1;        // a = m * 2^E, 1 <= m < 2
    const float m = __builtin_amdgcn_frexp_mantf(a) * 2.0f;  // exact
    e = E - 8 + (m > 1.75f ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const float f0 = __builtin_ldexpf(bf16_lo(v[i][j]), -e), f1 = __builtin_ldexpf(bf16_hi(v[i][j]), -e);
      const float f2 = __builtin_ldexpf(bf16_lo(v[i][j + 1]), -e), f3 = __builtin_ldexpf(bf16_hi(v[i][j + 1]), -e);
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, w, true);
      out[i / 2][(i % 2) * 2 + j / 2] = (uint32_t)w;
    }
  }
  return e;
}

// ---------------------------------------------------------------------------
// Misc
// ---------------------------------------------------------------------------
// silu(g) * u in FP32 with the hardware exponential and reciprocal (about 1 ulp each;
// the result is rounded to BF16, 2^16 times coarser). A correctly rounded division
// expands to about ten instructions per element, a large share of the GEMM epilogue.
// 1 + exp(-g) >= 1, so the reciprocal never sees a denormal; -g large gives +inf,
// whose reciprocal is 0, as the division would give.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <typename T>
__device__ __forceinline__ T ld_nt(const T* p) { return __builtin_nontemporal_load(p); }

}  // namespace moe4
