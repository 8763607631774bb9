// Grouped W4A16 expert FFN for few rows per expert (decode and batched decode).
//
// Decode is bound by reading the touched experts' weights once (the GB10 bandwidth
// budget article, section "Mechanism: decode is bandwidth-bound, prefill is
// compute-bound"); batching raises throughput by sharing each weight read across
// the rows of the batch (same article, "Batching changes the arithmetic"). So the
// kernel streams every touched tile once per 16 rows of its expert and nothing else
// from HBM.
//
// Weights are in the tiled layout (prepack.hip): a 16-row x 128-column tile is 1 KB
// of codes + 128 B of scales, stored in the lane order of the 16x16x32 BF16 MFMA
// operand, so each wave reads a tile with one contiguous 1 KB load and one 128 B load.
//
// Work split. A wave owns a pair of 16-row blocks (up: a gate block and the matching
// up block, so SwiGLU is applied in registers; down: two consecutive W2 blocks) and
// streams them along K. When the routing leaves too few blocks to fill the chip
// (ksplit > 1), the K range of a pair is split over ksplit waves of the workgroup,
// and their partial sums are added in a fixed order through LDS. Empty experts exit
// at once. Each K step is dequantised exactly into BF16 (code * E4M3 scale has at
// most 6 significant bits) in registers; the next two steps' tiles are already in
// flight. More than 16 rows of one expert take further passes over its tiles.
// When T*k < E, workgroups are launched only for as many experts as can have rows
// and each finds its expert among the non-empty ones from the offsets.
#include <algorithm>

#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

struct DecodeArgs {
  const uint16_t* act;      // up: x [T][H]; down: h [R][I]
  const int32_t* offsets;   // [G+1] or NULL (dense: one group of T rows)
  const int32_t* perm_src;  // up only: row -> flat pair (token = pair / k); NULL = identity
  int k;
  int T;
  const uint8_t* tcodes;    // tiled codes of [G][N][K]
  const uint8_t* tscales;   // tiled scales
  const float* tscale;      // [G]
  int N, K, I;              // up: N = 2I, K = H; down: N = H, K = I
  int ksplit;               // waves per pair along K: 1, 2 or 4
  uint16_t* out;            // up: h [R][I]; down: y [R][N]
  int G;                    // experts in the weight tensor
  int compact;              // grid rows index the non-empty experts (T*k < G)
};

constexpr int kSlices = 4;  // fixed K slices (see the accumulation order below)

struct Tile {
  u32x4 c0, c1;        // codes of the two blocks
  uint32_t s0, s1;     // two E4M3 scales per block (low half of the loaded dword)
};

__device__ __forceinline__ void load_tile(Tile& t, const uint8_t* c0, const uint8_t* c1, const uint8_t* s0,
                                          const uint8_t* s1, int lane) {
  t.c0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c0) + lane);
  t.c1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c1) + lane);
  t.s0 = reinterpret_cast<const uint16_t*>(s0)[lane];
  t.s1 = reinterpret_cast<const uint16_t*>(s1)[lane];
}

// The j-th expert (in index order) that has rows, or -1: a wave-wide ballot scan of
// the offsets, so workgroups are spent only on experts the routing touched.
__device__ __forceinline__ int nth_active_group(const int32_t* offsets, int G, int j) {
  const int lane = threadIdx.x & 63;
  int seen = 0;
  for (int base = 0; base < G; base += 64) {
    const int e = base + lane;
    const bool act = e < G && offsets[e + 1] > offsets[e];
    const uint64_t bal = __ballot(act);
    const int cnt = __popcll(bal);
    if (j < seen + cnt) {
      // position of the (j - seen)-th set bit
      uint64_t b = bal;
      for (int i = 0; i < j - seen; ++i) b &= b - 1;
      return base + __ffsll((long long)b) - 1;
    }
    seen += cnt;
  }
  return -1;
}

template <bool kUp>
__global__ __launch_bounds__(256, 4) void ffn_decode_kernel(DecodeArgs a) {
  __shared__ float4 red[2][kSlices][2][64];
  int g = blockIdx.y, r0 = 0, M = a.T;
  if (a.offsets) {
    if (a.compact) {
      g = nth_active_group(a.offsets, a.G, blockIdx.y);
      if (g < 0) return;
    }
    r0 = a.offsets[g];
    M = a.offsets[g + 1] - r0;
  }
  if (M <= 0) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rn = lane & 15, kq = lane >> 4;
  const int ksplit = a.ksplit, pairs = 4 / ksplit;
  const int p = wave / ksplit, q = wave % ksplit;
  const int K = a.K, NS = K / 128, NB = a.N / 16;
  // the pair's two blocks (row-block indices within the expert)
  int b0, b1, col0;
  if (kUp) {
    col0 = (blockIdx.x * pairs + p) * 16;  // h columns col0..col0+15
    b0 = col0 / 16;
    b1 = (a.I + col0) / 16;
  } else {
    col0 = (blockIdx.x * pairs + p) * 32;  // y columns col0..col0+31
    b0 = col0 / 16;
    b1 = b0 + 1;
  }
  const size_t tile0 = ((size_t)g * NB + b0) * NS, tile1 = ((size_t)g * NB + b1) * NS;
  // K is cut into kSlices fixed slices whose partial sums are always added as
  // ((s0 + s1) + s2) + s3, whichever waves computed them: the bits of a row do not
  // depend on ksplit, i.e. on how many tokens share the call.
  const int nsl = kSlices / ksplit, first = q * nsl;
  const int s_begin = first * NS / kSlices, s_end = (first + nsl) * NS / kSlices;
  const float ts = a.tscale[g];

  for (int pass = 0; pass < M; pass += 16) {
    // this lane's activation row (A operand row rn)
    const int m = pass + rn;
    const bool aval = m < M;
    const int r = r0 + (aval ? m : 0);
    int src = r;
    if (kUp) src = a.perm_src ? a.perm_src[r] / a.k : r;
    const uint16_t* arow = a.act + (size_t)src * K + kq * 32;

    // acc: the running slice; tot: slices first..current, summed in order (wave q = 0)
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, tot0 = acc0, tot1 = acc0;
    Tile t0, t1, t2;
    u32x4 xa[4];
    auto issue = [&](Tile& t, int s) {
      if (s < s_end)
        load_tile(t, a.tcodes + (tile0 + s) * 1024, a.tcodes + (tile1 + s) * 1024,
                  a.tscales + (tile0 + s) * 128, a.tscales + (tile1 + s) * 128, lane);
    };
    // rows past the expert's end read a valid row (r0) and are zeroed without a branch
    const uint32_t xmask = aval ? ~0u : 0u;
    auto load_x = [&](u32x4* xv, int s) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(arow + s * 128 + 8 * j);
        xv[j] = u32x4{v[0] & xmask, v[1] & xmask, v[2] & xmask, v[3] & xmask};
      }
    };
    // close slice `sl`: wave 0 adds it to its running total; other waves hand it over
    auto close_slice = [&](int sl) {
      if (q == 0) {
        tot0 += acc0;
        tot1 += acc1;
      } else {
        red[p][sl][0][lane] = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
        red[p][sl][1][lane] = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
      }
      acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1 = acc0;
    };
    issue(t0, s_begin);
    issue(t1, s_begin + 1);
    int sl = first;
    while (sl < first + nsl && (sl + 1) * NS / kSlices <= s_begin) close_slice(sl++);  // empty slices
    for (int s = s_begin; s < s_end; ++s) {
      issue(t2, s + 2);
      load_x(xa, s);
      const float sa0 = e4m3_to_f32<0>(t0.s0), sa1 = e4m3_to_f32<1>(t0.s0);
      const float sb0 = e4m3_to_f32<0>(t0.s1), sb1 = e4m3_to_f32<1>(t0.s1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = mfma16x16x32(xa[j], dequant8(t0.c0[j], j < 2 ? sa0 : sa1), acc0);
        acc1 = mfma16x16x32(xa[j], dequant8(t0.c1[j], j < 2 ? sb0 : sb1), acc1);
      }
      t0 = t1;
      t1 = t2;
      // close every slice that ends here (a slice is empty when NS < 4)
      while (sl < first + nsl && (sl + 1) * NS / kSlices <= s + 1) close_slice(sl++);
    }
    while (sl < first + nsl) close_slice(sl++);

    if (ksplit > 1) {
      __syncthreads();
      if (q == 0) {
        for (int w = nsl; w < kSlices; ++w) {  // the other waves' slices, in order
          const float4 u0 = red[p][w][0][lane], u1 = red[p][w][1][lane];
          tot0[0] += u0.x; tot0[1] += u0.y; tot0[2] += u0.z; tot0[3] += u0.w;
          tot1[0] += u1.x; tot1[1] += u1.y; tot1[2] += u1.z; tot1[3] += u1.w;
        }
      }
      __syncthreads();
    }
    if (q == 0) {
      const int mbase = pass + 4 * kq;  // rows mbase..mbase+3, column rn
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mbase + i < M) {
          uint16_t* orow;
          if (kUp) {
            orow = a.out + (size_t)(r0 + mbase + i) * a.I + col0 + rn;
            orow[0] = f32_to_bf16(silu_mul(ts * tot0[i], ts * tot1[i]));
          } else {
            orow = a.out + (size_t)(r0 + mbase + i) * a.N + col0 + rn;
            orow[0] = f32_to_bf16(ts * tot0[i]);
            orow[16] = f32_to_bf16(ts * tot1[i]);
          }
        }
      }
    }
  }
}

// Waves per pair along K: enough waves to fill the chip when few pairs are active.
int pick_ksplit(long long active_groups, long long pairs_per_group) {
  const long long pairs = active_groups * pairs_per_group;
  if (pairs >= 4096) return 1;
  if (pairs >= 1024) return 2;
  return 4;
}

hipError_t launch(bool up, const DecodeArgs& base, long long active_groups, int G, hipStream_t s) {
  DecodeArgs a = base;
  const long long pairs_per_group = up ? a.I / 16 : a.N / 32;
  a.ksplit = pick_ksplit(active_groups, pairs_per_group);
  const int per_wg = 4 / a.ksplit;
  a.G = G;
  // when fewer experts can have rows than exist, one grid row per possible one
  a.compact = active_groups < G;
  dim3 grid((unsigned)(pairs_per_group / per_wg), (unsigned)(a.compact ? active_groups : G));
  if (up) hipLaunchKernelGGL(ffn_decode_kernel<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(ffn_decode_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_decode(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                         int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  DecodeArgs a{x, offsets, perm_src, k, T, w13.packed, w13.scales, w13.tscale, 2 * I, H, I, 1, h, G, 0};
  const long long active = offsets ? std::min<long long>((long long)T * k, G) : 1;
  return launch(true, a, active, G, s);
}

hipError_t launch_ffn_down_decode(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H, int I,
                           W4View w2, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  DecodeArgs a{h, offsets, nullptr, 1, T, w2.packed, w2.scales, w2.tscale, H, I, I, 1, y, G, 0};
  const long long active = offsets ? std::min<long long>((long long)T * k, G) : 1;
  return launch(false, a, active, G, s);
}

}  // namespace moe4
