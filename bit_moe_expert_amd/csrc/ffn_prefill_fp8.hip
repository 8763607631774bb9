// The FP8 form (W4A8) of the prefill grouped GEMM: activations as block-scaled E4M3
// (32 values per E8M0 scale, quant.hip), weights dequantised and rounded to E4M3,
// gfx950's block-scaled 32x32x64 FP8 MFMA (twice the BF16 rate). The structure is the BF16 kernel's: four
// waves, each owning all 256 rows of 64 columns; every load a direct-to-LDS copy in a
// three-slot ring; one barrier per K step before its last substep, which fetches the
// next step's first operands. A K step is 128 (one 128-byte activation row, one
// 128-column weight tile), two substeps of K = 64.
//
// MFMA operands (as measured on gfx950): lane l supplies row (A) or column (B) l%32;
// its bytes 0..15 hold K = 16hh .. +15 of the instruction's first 32-wide K block and
// bytes 16..31 the same of the second (hh = l/32), and the A scale of lane m + 32b is
// the E8M0 scale of row m's block b. An activation block of 32 is exactly one such K
// block, so block scaling costs nothing: the lane reads 16-byte chunks 4ks + hh and
// 4ks + 2 + hh of the step's row and passes block 2ks + hh's scale. The weight lane
// reads one lane of the tiled layout (row rn, 32-column quarter kq = 2ks + hh: 16 code
// bytes, the E4M3 scales of its two 16-groups) and trades its second group for the
// first group of lane l ^ 32 (v_permlane32_swap) to reach the same K order; each
// code * scale is formed in FP16 (exact) and rounded to E4M3 (nearest even; products
// above 448, possible only with block scales above 74, are clamped to 448 first, the
// reading's saturation).
#include "prefill_common.hpp"

namespace moe4 {

namespace {

using namespace prefill;

constexpr int BK8 = 128;                          // K per step
constexpr int kBWave8 = 2 * 2048 + 2 * 256;       // weight bytes one wave copies per step

typedef int v8i32 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i32 cat8(u32x4 lo, u32x4 hi) {
  v8i32 r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// 32 E2M1 codes (4 dwords) of one weight row, times their two E4M3 scales (the low
// 2 bytes of sc: codes 0..15, then 16..31) -> 32 E4M3 bytes (8 dwords).
__device__ __forceinline__ v8i32 dequant32_fp8(u32x4 c, uint32_t sc) {
  const f16x2 s2 = e4m3x2_to_f16(sc);
  v8i32 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const _Float16 s = s2[d / 2];
    const f16x2 ss = {s, s};
    f16x2 p[4];
    p[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 0) * ss;
    p[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 1) * ss;
    p[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 2) * ss;
    p[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 3) * ss;
    {  // saturate at 448
      const f16x2 hi = {(_Float16)448.0f, (_Float16)448.0f}, lo = {(_Float16)-448.0f, (_Float16)-448.0f};
#pragma unroll
      for (int q = 0; q < 4; ++q) p[q] = __builtin_elementwise_max(__builtin_elementwise_min(p[q], hi), lo);
    }
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    s16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(s16x2{0, 0}, p[0], 1.0f, false);
    w0 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w0, p[1], 1.0f, true);
    s16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(s16x2{0, 0}, p[2], 1.0f, false);
    w1 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w1, p[3], 1.0f, true);
    r[2 * d] = __builtin_bit_cast(int, w0);
    r[2 * d + 1] = __builtin_bit_cast(int, w1);
  }
  return r;
}

// The same through a table: for each E4M3 scale byte, the E4M3 bytes of the eight E2M1
// magnitudes (0, 0.5, 1, 1.5, 2, 3, 4, 6) times that scale, formed once per workgroup
// by dequant32_fp8 itself (so every byte, saturation included, is the same). A dword of
// codes (eight weights sharing one scale) then takes two byte permutes for the
// magnitudes of its even and odd nibbles, the codes' sign bits XOR-ed in (E4M3 and
// E2M1 both keep the sign in the top bit, and a negative scale's entries carry its
// sign), and two byte permutes back into element order: about 10 instructions per 8
// weights instead of 20. (A NaN scale byte, 0x7f or 0xff, gives +-448 by the code's
// sign.)
__device__ __forceinline__ v8i32 dequant32_fp8_lut(u32x4 c, uint32_t sc, const uint32_t* tab) {
  const uint2 t0 = *reinterpret_cast<const uint2*>(tab + 2 * (sc & 0xffu));
  const uint2 t1 = *reinterpret_cast<const uint2*>(tab + 2 * ((sc >> 8) & 0xffu));
  v8i32 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint2 t = d < 2 ? t0 : t1;
    const uint32_t w = c[d];
    // elements 0, 2, 4, 6 (low nibbles) and 1, 3, 5, 7 (high nibbles), one a byte
    const uint32_t ev = __builtin_amdgcn_perm(t.y, t.x, w & 0x07070707u) ^ ((w << 4) & 0x80808080u);
    const uint32_t od = __builtin_amdgcn_perm(t.y, t.x, (w >> 4) & 0x07070707u) ^ (w & 0x80808080u);
    r[2 * d] = (int)__builtin_amdgcn_perm(od, ev, 0x05010400u);      // elements 0..3
    r[2 * d + 1] = (int)__builtin_amdgcn_perm(od, ev, 0x07030602u);  // elements 4..7
  }
  return r;
}

__device__ __forceinline__ f32x16 mfma_fp8(v8i32 a, v8i32 b, int sa, f32x16 c) {
  // A and B both E4M3 (format 0); A block scale sa (E8M0), B scale 2^0 (127)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, 127);
}

template <bool kUp, bool kDense, bool kTiled>
__global__ __launch_bounds__(kThreads, 1) void ffn_prefill_fp8_kernel(GemmArgs a) {
  // activation ring [256][128] E4M3, their scale ring ([4 waves][64 rows] dwords),
  // weight ring (per wave: two blocks of two 1 KB tiles of codes, then their scales)
  __shared__ __attribute__((aligned(16))) uint8_t lds0[BM * BK8];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[BM * BK8];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[BM * BK8];
  __shared__ __attribute__((aligned(16))) uint32_t ldss0[4 * 64];
  __shared__ __attribute__((aligned(16))) uint32_t ldss1[4 * 64];
  __shared__ __attribute__((aligned(16))) uint32_t ldss2[4 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb0[4 * kBWave8];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb1[4 * kBWave8];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb2[4 * kBWave8];
  __shared__ int sched[4];
  __shared__ __attribute__((aligned(16))) uint32_t ldst[2 * 256];  // E4M3 table per scale byte

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) tile_schedule<kDense>(a, lane, sched);
  static_assert(kThreads == 256, "one thread per table entry (scale byte)");
  {  // thread t forms the table entry of scale byte t: codes 0..7 (magnitudes) times it
    const v8i32 e = dequant32_fp8(u32x4{0x76543210u, 0u, 0u, 0u}, (uint32_t)tid | ((uint32_t)tid << 8));
    *reinterpret_cast<uint2*>(&ldst[2 * tid]) = make_uint2((uint32_t)e[0], (uint32_t)e[1]);
  }
  __syncthreads();
  const int g = sched[0];
  if (g < 0) return;
  const int nt = sched[3];
  const int row0 = sched[1], rows = sched[2];

  const int K = a.K, NS = K / 128, NB = a.N / 16, nsteps = K / BK8, KS = K / 32;
  const float ts = a.tscale[g];
  const int r32 = lane & 31, hh = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // weight copy sources of block j (32 rows): two 16-row tiles, this lane's 16 code
  // bytes and scale dword of each step, arranged in LDS as the tiled layout's lanes
  // (row rn, 32-column quarter kq at (rn + 16 kq) * 16) for both layouts
  const uint8_t* bsrc[2][2];
  const uint8_t* ssrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n0 = kUp ? (j == 0 ? nt * 128 + 32 * wv : a.I + nt * 128 + 32 * wv) : nt * BN + 64 * wv + 32 * j;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (kTiled) {
        bsrc[j][t] = a.tcodes + ((size_t)g * NB + n0 / 16 + t) * NS * 1024 + lane * 16;
      } else {
        bsrc[j][t] = a.tcodes + ((size_t)g * a.N + n0 + 16 * t + (lane & 15)) * (K / 2) + (lane >> 4) * 16;
      }
    }
    const int t = lane >> 5, l2 = lane & 31;
    if constexpr (kTiled) {
      ssrc[j] = a.tscales + ((size_t)g * NB + n0 / 16 + t) * NS * 128 + l2 * 4;
    } else {  // two dwords of each row's 8 scale bytes of a step: LDS [16 rows][8 bytes]
      ssrc[j] = a.tscales + ((size_t)g * a.N + n0 + 16 * t + (l2 >> 1)) * (K / 16) + (l2 & 1) * 4;
    }
  }

  auto compute = [&](auto MIC) {
    constexpr int MI = decltype(MIC)::value;
    constexpr int RW = 8 * MI;
    // activation rows: wave w copies rows RW*w .. +RW-1, 8 a copy, chunks swizzled
    const uint8_t* asrc[8];  // (sized by the most MI: see the BF16 kernel)
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int rr = RW * wv + 8 * i + (lane >> 3);
      int src = row0 + (rr < rows ? rr : 0);
      if (kUp && !kDense) src = a.perm_src[src] / a.k;
      asrc[i] = a.act8 + (size_t)src * K + (((lane & 7) ^ swz_key(rr)) << 4);
    }
    // block scales of the wave's rows: lane l copies row RW*w + min(l, RW-1)'s four
    // scale bytes of the step into dword l of the wave's 64
    const uint8_t* scsrc;
    {
      const int rr = RW * wv + (lane < RW ? lane : RW - 1);
      int src = row0 + (rr < rows ? rr : 0);
      if (kUp && !kDense) src = a.perm_src[src] / a.k;
      scsrc = a.ascale + (size_t)src * KS;
    }
    auto abuf = [&](auto RC) -> uint8_t* {
      constexpr int R = decltype(RC)::value;
      return R == 0 ? lds0 : (R == 1 ? lds1 : lds2);
    };
    auto sbuf = [&](auto RC) -> uint32_t* {
      constexpr int R = decltype(RC)::value;
      return R == 0 ? ldss0 : (R == 1 ? ldss1 : ldss2);
    };
    auto bbuf = [&](auto RC) -> uint8_t* {
      constexpr int R = decltype(RC)::value;
      return (R == 0 ? ldsb0 : (R == 1 ? ldsb1 : ldsb2)) + wv * kBWave8;
    };
    auto load = [&](int st, uint8_t* ab, uint32_t* sb, uint8_t* bb) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const uint8_t* src = asrc[i] + st * BK8;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)&ab[(RW * wv + 8 * i) * BK8],
                                         16, 0, 0);
      }
      const uint8_t* ssp = scsrc + st * 4;
      __builtin_amdgcn_global_load_lds(ssp, (__attribute__((address_space(3))) void*)&sb[64 * wv], 4, 0, 0);
      const size_t co = kTiled ? (size_t)st * 1024 : (size_t)st * 64;
      const size_t so = kTiled ? (size_t)st * 128 : (size_t)st * 8;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint8_t* cp = bsrc[j][t] + co;
          __builtin_amdgcn_global_load_lds(cp, (__attribute__((address_space(3))) void*)(bb + j * 2048 + t * 1024),
                                           16, 0, 0);
        }
        const uint8_t* sp = ssrc[j] + so;
        __builtin_amdgcn_global_load_lds(sp, (__attribute__((address_space(3))) void*)(bb + 4096 + j * 256), 4, 0, 0);
      }
    };
    f32x16 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int key = swz_key(r32);
    const int rn = r32 & 15, tt = r32 >> 4;
    // byte selector of the swapped scale pair (v_perm_b32: 0-3 the first swap result,
    // 4-7 the second, 0x0c a zero byte): l < 32 (own b0, partner b0), l >= 32
    // (partner b1, own b1)
    const uint32_t ssel = hh ? 0x0c0c0501u : 0x0c0c0400u;
    // operands of substep ks: A fragments (32 bytes of row 32i + r32), A block scales,
    // dequantised weight fragments
    auto read_ops = [&](auto RC, int ks, v8i32* A, int* SA, v8i32* Bv) {
      const uint8_t* ab = abuf(RC);
      const uint32_t* sb = sbuf(RC);
      const uint8_t* bb = bbuf(RC);
      const int c0 = ((4 * ks + hh) ^ key) << 4, c1 = ((4 * ks + 2 + hh) ^ key) << 4;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = 32 * i + r32;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&ab[row * BK8 + c0]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&ab[row * BK8 + c1]);
        A[i] = cat8(lo, hi);
        // the row's scale dword: wave row / RW copied it, to position row % RW
        const uint32_t sw = sb[64 * (row / RW) + row % RW];
        SA[i] = (int)((sw >> (8 * (2 * ks + hh))) & 0xffu);
      }
      const int kq = 2 * ks + hh;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(bb + j * 2048 + tt * 1024 + (rn + 16 * kq) * 16);
        const int soff = kTiled ? (rn + 16 * kq) * 2 : rn * 8 + 2 * kq;
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(bb + 4096 + j * 256 + tt * 128 + soff);
        // lane l < 32 keeps groups 0 and takes the partner's group 0; lane l >= 32 takes
        // the partner's group 1 and keeps its own
        const auto s0 = __builtin_amdgcn_permlane32_swap(c[0], c[2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(c[1], c[3], false, false);
        const u32x4 cs = {s0[0], s1[0], s0[1], s1[1]};
        const auto ss = __builtin_amdgcn_permlane32_swap(sc, sc, false, false);
        Bv[j] = dequant32_fp8_lut(cs, __builtin_amdgcn_perm(ss[1], ss[0], ssel), ldst);
      }
    };
    constexpr int kAfter = MI + 7;  // one step's copies: MI rows, 1 scale, 4 codes, 2 scales
    constexpr int kWait = (kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (0 << 8);
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    v8i32 fa[MI], fb[2];
    int fsa[MI];
    load(0, abuf(C0{}), sbuf(C0{}), bbuf(C0{}));
    load(min(1, nsteps - 1), abuf(C1{}), sbuf(C1{}), bbuf(C1{}));
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("s_barrier" ::: "memory");
    read_ops(C0{}, 0, fa, fsa, fb);
    auto step = [&](auto RC, int st) {
      constexpr int R = decltype(RC)::value;
      using CR1 = std::integral_constant<int, (R + 1) % 3>;
      using CR2 = std::integral_constant<int, (R + 2) % 3>;
      const int nx = min(st + 2, nsteps - 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8i32 na[MI], nb[2];
        int nsa[MI];
        if (ks == 0) {
          load(nx, abuf(CR2{}), sbuf(CR2{}), bbuf(CR2{}));
          read_ops(RC, 1, na, nsa, nb);
        } else {
          // every wave's copies of step st+1 have landed, and every wave is past its
          // reads of step st-1's slot (refilled at the next step's start)
          __builtin_amdgcn_s_waitcnt(kWait);
          asm volatile("s_barrier" ::: "memory");
          read_ops(CR1{}, 0, na, nsa, nb);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma_fp8(fa[i], fb[j], fsa[i], acc[i][j]);
#pragma unroll
        for (int g2 = 0; g2 < 2 * MI; ++g2) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          if (ks == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (copies)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          fa[i] = na[i];
          fsa[i] = nsa[i];
        }
        fb[0] = nb[0];
        fb[1] = nb[1];
      }
    };
    int st = 0;
    for (const int st_end = nsteps - nsteps % 3; st < st_end; st += 3) {
      step(C0{}, st);
      step(C1{}, st + 1);
      step(C2{}, st + 2);
    }
    if (st < nsteps) step(C0{}, st);
    if (st + 1 < nsteps) step(C1{}, st + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- epilogue (acc[i][j][r]: row 32i + 8(r/4) + 4hh + r%4, column r32 of block j) ----
    // staged through LDS as BF16 ([rows][W], wave w in the first or second half of
    // ring slot w/2, in two halves of the rows for down)
    constexpr int W = kUp ? 32 : 64;
    uint16_t* stage = reinterpret_cast<uint16_t*>((wv < 2 ? lds0 : lds1) + (wv & 1) * 16384);
    const size_t ld = kUp ? a.I : a.N;
    const int col0 = kUp ? nt * 128 + 32 * wv : nt * BN + 64 * wv;
    constexpr int kHalves = kUp ? 1 : 2;  // down: at most 128 rows of 64 columns at a time
    constexpr int B0 = (MI + kHalves - 1) / kHalves;  // 32-row blocks of the first half
    constexpr int HR = 32 * B0;                        // rows of the first half
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
#pragma unroll
      for (int i = half * B0; i < (half == 0 ? B0 : MI); ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3) - half * HR;
          if (kUp) {
            stage[lr * W + r32] = f32_to_bf16(silu_mul(ts * acc[i][0][r], ts * acc[i][1][r]));
          } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) stage[lr * W + 32 * j + r32] = f32_to_bf16(ts * acc[i][j][r]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (a.out != nullptr) {  // BF16 rows (y for down; h for up when asked for)
        const int kPieces = 32 * (half == 0 ? B0 : MI - B0) * W / 8;  // a multiple of 64
#pragma unroll
        for (int c = 0; c < kPieces / 64; ++c) {
          const int piece = 64 * c + lane, lr = piece / (W / 8), lc = (piece % (W / 8)) * 8;
          const int tr = half * HR + lr;
          if (tr < rows)
            *reinterpret_cast<u32x4*>(a.out + (size_t)(row0 + tr) * ld + col0 + lc) =
                *reinterpret_cast<const u32x4*>(stage + lr * W + lc);
        }
      }
      if constexpr (kUp) {
        // h for the down projection: each row's 32 columns are one FP8 block
#pragma unroll
        for (int c = 0; c < (32 * MI + 63) / 64; ++c) {
          const int lr = 64 * c + lane;
          if (lr < 32 * MI && lr < rows) {
            u32x4 v[4], q[2];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const u32x4*>(stage + lr * W + 8 * u);
            const int e = mxfp8_block(v, q);
            u32x4* dst = reinterpret_cast<u32x4*>(a.out8 + (size_t)(row0 + lr) * a.I + col0);
            dst[0] = q[0];
            dst[1] = q[1];
            a.oscale[(size_t)(row0 + lr) * (a.I / 32) + col0 / 32] = (uint8_t)(e + 127);
          }
        }
      }
      if (half + 1 < kHalves) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  };
  // 32-row blocks a wave computes: the tile's rows rounded up to 32 (2 to 8)
  if (rows <= 64) compute(std::integral_constant<int, 2>{});
  else if (rows <= 96) compute(std::integral_constant<int, 3>{});
  else if (rows <= 128) compute(std::integral_constant<int, 4>{});
  else if (rows <= 160) compute(std::integral_constant<int, 5>{});
  else if (rows <= 192) compute(std::integral_constant<int, 6>{});
  else if (rows <= 224) compute(std::integral_constant<int, 7>{});
  else compute(std::integral_constant<int, 8>{});
}


hipError_t launch_fp8(bool up, GemmArgs a, long long m_tiles, hipStream_t s) {
  const dim3 g = size_grid(a, up, m_tiles), b(kThreads);
  const bool dense = a.offsets == nullptr;
  if (a.tiled) {
    if (!dense && up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<true, false, true>), g, b, 0, s, a);
    if (!dense && !up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<false, false, true>), g, b, 0, s, a);
    if (dense && up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<true, true, true>), g, b, 0, s, a);
    if (dense && !up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<false, true, true>), g, b, 0, s, a);
  } else {
    if (!dense && up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<true, false, false>), g, b, 0, s, a);
    if (!dense && !up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<false, false, false>), g, b, 0, s, a);
    if (dense && up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<true, true, false>), g, b, 0, s, a);
    if (dense && !up) hipLaunchKernelGGL((ffn_prefill_fp8_kernel<false, true, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_prefill_fp8(const uint8_t* x8, const uint8_t* xs, const int32_t* offsets,
                                     const int32_t* perm_src, int k, int T, int G, int H, int I, W4View w13,
                                     uint16_t* h, uint8_t* h8, uint8_t* hs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{nullptr, offsets, perm_src, k, T, w13.packed, w13.scales, w13.tscale, 2 * I, H, I, G, h, 0, 0,
             w13.tiled ? 1 : 0, x8, xs, h8, hs};
  return launch_fp8(true, a, m_tile_bound(offsets, T, k, G), s);
}

hipError_t launch_ffn_down_prefill_fp8(const uint8_t* h8, const uint8_t* hs, const int32_t* offsets, int k, int T,
                                       int G, int H, int I, W4View w2, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{nullptr, offsets, nullptr, 1, T, w2.packed, w2.scales, w2.tscale, H, I, I, G, y, 0, 0,
             w2.tiled ? 1 : 0, h8, hs, nullptr, nullptr};
  return launch_fp8(false, a, m_tile_bound(offsets, T, k, G), s);
}

}  // namespace moe4
