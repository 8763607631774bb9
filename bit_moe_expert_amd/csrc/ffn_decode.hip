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

// One K step of a wave: its two 16 x 128 weight tiles and, when the activations are
// not staged in LDS, its activation fragment.
template <bool kXLds>
struct Stage {
  u32x4 c0, c1;     // codes of the two blocks (this lane's 16 bytes of each 1 KB tile)
  uint32_t s0, s1;  // two E4M3 scales per block (low half of the loaded dword)
  u32x4 x[4];       // activation row rn, columns 128s + 32kq .. +31
};
template <>
struct Stage<true> {
  u32x4 c0, c1;
  uint32_t s0, s1;
};

// The expert a workgroup works on and its rows [r0, r0 + M).
struct Group {
  int g, r0, M;
};

// Grid row j -> group. Compact grids (T*k < G) take the j-th expert (in index order)
// that has rows, found from one round of loads: lane l looks at experts 4l .. 4l+3
// (G <= 256), a wave scan of the per-lane counts finds the lane holding the j-th,
// and that lane's expert and row range are broadcast. M = 0 if there is none.
__device__ __forceinline__ Group find_group(const DecodeArgs& a) {
  const int j = blockIdx.y;
  if (!a.offsets) return Group{0, 0, a.T};
  if (!a.compact) {
    const int r0 = a.offsets[j];
    return Group{j, r0, a.offsets[j + 1] - r0};
  }
  const int lane = threadIdx.x & 63;
  const int G = a.G;
  int v[5];
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    const int e = 4 * lane + c;
    v[c] = e <= G ? a.offsets[e] : 0;
  }
  bool act[4];
  int cnt = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    act[c] = 4 * lane + c < G && v[c + 1] > v[c];
    cnt += act[c] ? 1 : 0;
  }
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int excl = incl - cnt;
  const uint64_t bal = __ballot(j >= excl && j < incl);
  if (bal == 0) return Group{0, 0, 0};
  int g = 0, r0 = 0, M = 0, need = j - excl;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (act[c]) {
      if (need == 0) {
        g = 4 * lane + c;
        r0 = v[c];
        M = v[c + 1] - v[c];
      }
      --need;
    }
  }
  const int owner = __ffsll((long long)bal) - 1;
  return Group{__builtin_amdgcn_readlane(g, owner), __builtin_amdgcn_readlane(r0, owner),
               __builtin_amdgcn_readlane(M, owner)};
}

// Byte stride of one activation row staged in LDS: 16 bytes of padding shift
// consecutive rows by four banks, so the 16 rows of an MFMA operand read conflict-free.
__host__ __device__ constexpr int x_row_stride(int K) { return 2 * K + 16; }

// The kernel. D = K steps in the register ring: while step s is multiplied, steps
// s+1 .. s+D-1 are in flight. Loads are never skipped (past the end they re-read the
// last step), so the number of loads in flight is the same on every path and the
// compiler's wait counts stay at D-1 stages.
//
// kXLds: the workgroup first copies its rows' activations (rows_alloc rows x K) into
// LDS and the waves read their MFMA operand from there; this frees the 16 registers
// per stage that the fragment otherwise takes, so more weight tiles are in flight.
// It is used when the rows of a pass fit in a few tens of KB of LDS (decode batches).
template <bool kUp, int D, bool kXLds>
__global__ __launch_bounds__(256, 4) void ffn_decode_kernel(DecodeArgs a,
                                                                                      int rows_alloc) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Group grp = find_group(a);
  const int g = grp.g, r0 = grp.r0, M = grp.M;
  if (M <= 0) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar registers)
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
  // each block's K tiles through a buffer resource covering exactly those tiles, so
  // a step needs one offset register and an access past them would read zeros
  const BufRes rc0 = make_res(a.tcodes + tile0 * 1024, NS * 1024);
  const BufRes rc1 = make_res(a.tcodes + tile1 * 1024, NS * 1024);
  const BufRes rs0 = make_res(a.tscales + tile0 * 128, NS * 128);
  const BufRes rs1 = make_res(a.tscales + tile1 * 128, NS * 128);
  // K is cut into kSlices fixed slices whose partial sums are always added as
  // ((s0 + s1) + s2) + s3, whichever waves computed them: the bits of a row do not
  // depend on ksplit, i.e. on how many tokens share the call.
  const int nsl = kSlices / ksplit, first = q * nsl;
  const int s_begin = first * NS / kSlices, s_end = (first + nsl) * NS / kSlices;
  const float ts = a.tscale[g];
  const int xs = x_row_stride(K);
  // slices of waves q > 0 handed to wave 0: [pairs][kSlices - nsl][2][64] float4,
  // after the staged activations when those are in LDS
  float4* red = reinterpret_cast<float4*>(smem + (kXLds ? (size_t)rows_alloc * xs : 0));
  const int rows_per_pass = kXLds ? rows_alloc : 16;

  for (int pass = 0; pass < M; pass += rows_per_pass) {
    const int nr = min(rows_per_pass, M - pass);  // real rows in this pass
    // rows past the pass's real rows use the pass's first row: MFMA rows are
    // independent and those rows are not stored
    const int m = rn < nr ? rn : 0;

    Stage<kXLds> st[D];
    const uint16_t* arow = nullptr;
    if (!kXLds) {
      const int r = r0 + pass + m;
      const int src = kUp && a.perm_src ? a.perm_src[r] / a.k : r;
      arow = a.act + (size_t)src * K + kq * 32;
    }
    // steps past the wave's range re-read its last step; a wave with an empty range
    // (NS < kSlices) reads step 0 and never uses it: every wave issues the same loads,
    // so the wait counts after them do not depend on the path taken
    auto issue = [&](Stage<kXLds>& t, int s) {
      s = s < s_end ? s : s_end - 1;
      s = s > 0 ? s : 0;
      const int co = s * 1024 + lane * 16, so = s * 128 + lane * 2;
      t.c0 = load_b128_nt(rc0, co);
      t.c1 = load_b128_nt(rc1, co);
      t.s0 = load_b16(rs0, so);
      t.s1 = load_b16(rs1, so);
      if constexpr (!kXLds) {
#pragma unroll
        for (int j = 0; j < 4; ++j) t.x[j] = *reinterpret_cast<const u32x4*>(arow + s * 128 + 8 * j);
      }
    };
    // lane i < 16 loads the source row of pass row i first: loads complete in issue
    // order, so this one does not wait behind the weight tiles issued next
    int row_src = 0;
    if (kXLds && lane < 16) {
      const int r = r0 + pass + (lane < nr ? lane : 0);
      row_src = kUp && a.perm_src ? a.perm_src[r] : r;
    }
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(st[i], s_begin + i);
    const bool has_steps = s_begin < s_end;
    if constexpr (kXLds) {
      // stage rows pass .. pass+nr-1 of the expert: row i of LDS <- its source row
      if (kUp && a.perm_src) row_src /= a.k;  // pair index -> token
      if (pass > 0) __syncthreads();  // the previous pass's reads are done
      const int cpr = K / 8;           // 16-byte chunks per row
      const int total = nr * cpr;
      for (int base = 0; base < total; base += 8 * 256) {
        u32x4 buf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = base + u * 256 + tid;
          const int row = c < total ? c / cpr : 0, col = c < total ? c % cpr : 0;
          const int sr = __shfl(row_src, row);
          buf[u] = reinterpret_cast<const u32x4*>(a.act + (size_t)sr * K)[col];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = base + u * 256 + tid;
          if (c < total) *reinterpret_cast<u32x4*>(smem + (size_t)(c / cpr) * xs + (c % cpr) * 16) = buf[u];
        }
      }
      __syncthreads();
    }
    const uint8_t* xl = smem + (size_t)m * xs + kq * 64;  // this lane's LDS operand row

    // acc: the running slice; tot: slices first..current, summed in order (wave q = 0)
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, tot0 = acc0, tot1 = acc0;
    auto compute = [&](const Stage<kXLds>& t, int s) {
      u32x4 xv[4];
      if constexpr (kXLds) {
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = *reinterpret_cast<const u32x4*>(xl + s * 256 + 16 * j);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[j] = t.x[j];
      }
      const float sa0 = e4m3_to_f32<0>(t.s0), sa1 = e4m3_to_f32<1>(t.s0);
      const float sb0 = e4m3_to_f32<0>(t.s1), sb1 = e4m3_to_f32<1>(t.s1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = mfma16x16x32(xv[j], dequant8(t.c0[j], j < 2 ? sa0 : sa1), acc0);
        acc1 = mfma16x16x32(xv[j], dequant8(t.c1[j], j < 2 ? sb0 : sb1), acc1);
      }
    };
    // close slice `sl`: wave 0 adds it to its running total; other waves hand it over
    auto close_slice = [&](int sl) {
      if (q == 0) {
        tot0 += acc0;
        tot1 += acc1;
      } else {
        float4* r = red + ((size_t)(p * (kSlices - nsl) + (sl - nsl)) * 2) * 64;
        r[lane] = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
        r[64 + lane] = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
      }
      acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1 = acc0;
    };
    int sl = first;
    if (has_steps) {
      while (sl < first + nsl && (sl + 1) * NS / kSlices <= s_begin) close_slice(sl++);  // empty slices
      for (int sb = s_begin; sb < s_end; sb += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          issue(st[(i + D - 1) % D], sb + i + D - 1);
          if (sb + i < s_end) {
            compute(st[i], sb + i);
            // close every slice that ends here (a slice is empty when NS < 4)
            while (sl < first + nsl && (sl + 1) * NS / kSlices <= sb + i + 1) close_slice(sl++);
          }
        }
      }
    }
    while (sl < first + nsl) close_slice(sl++);

    if (ksplit > 1) {
      __syncthreads();
      if (q == 0) {
        for (int w = nsl; w < kSlices; ++w) {  // the other waves' slices, in order
          const float4* r = red + ((size_t)(p * (kSlices - nsl) + (w - nsl)) * 2) * 64;
          const float4 u0 = r[lane], u1 = r[64 + lane];
          tot0[0] += u0.x; tot0[1] += u0.y; tot0[2] += u0.z; tot0[3] += u0.w;
          tot1[0] += u1.x; tot1[1] += u1.y; tot1[2] += u1.z; tot1[3] += u1.w;
        }
      }
      __syncthreads();
    }
    if (q == 0) {
      const int mbase = 4 * kq;  // pass rows mbase..mbase+3, column rn
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mbase + i < nr) {
          const size_t row = (size_t)(r0 + pass + mbase + i);
          if (kUp) {
            a.out[row * a.I + col0 + rn] = f32_to_bf16(silu_mul(ts * tot0[i], ts * tot1[i]));
          } else {
            uint16_t* orow = a.out + row * a.N + col0 + rn;
            orow[0] = f32_to_bf16(ts * tot0[i]);
            orow[16] = f32_to_bf16(ts * tot1[i]);
          }
        }
      }
    }
  }
}

constexpr int kStagesReg = 3;   // activation fragment in registers
constexpr int kStagesLds = 4;   // activations in LDS
constexpr int kWavesPerSimd = 4;  // both forms fit 128 VGPRs
constexpr size_t kXLdsMaxBytes = 40 * 1024;
constexpr size_t kLdsPerCu = 160 * 1024;

int cu_count() {
  static thread_local int cached_dev = -1, cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != cached_dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached_dev = dev;
    cached = n;
  }
  return cached;
}

hipError_t launch(bool up, const DecodeArgs& base, long long active_groups, int G, hipStream_t s) {
  DecodeArgs a = base;
  a.G = G;
  // when fewer experts can have rows than exist, one grid row per possible one
  a.compact = active_groups < G;
  const long long pairs_per_group = up ? a.I / 16 : a.N / 32;
  const long long pairs = active_groups * pairs_per_group;
  // staged rows: at most T (a token sends one row to an expert unless the caller's
  // routing repeats experts, which only adds passes)
  const int rows_alloc = a.T < 16 ? a.T : 16;
  const size_t x_bytes = (size_t)rows_alloc * x_row_stride(a.K);
  const bool use_lds = x_bytes <= kXLdsMaxBytes;
  // K split: the most waves per pair for which the whole grid is resident at once,
  // so that every wave starts in the first wave of dispatch and no second, partial
  // round of waves trails behind (a wave's lifetime is a few memory latencies)
  auto lds_bytes = [&](int ks) {
    const size_t red = ks > 1 ? (size_t)(4 / ks) * (kSlices - kSlices / ks) * 2 * 64 * 16 : 0;
    return (use_lds ? x_bytes : 0) + red;
  };
  auto resident_waves = [&](int ks) {
    const size_t lds = lds_bytes(ks);
    long long wg_per_cu = kWavesPerSimd;  // 4 waves per workgroup, one per SIMD
    if (lds > 0) wg_per_cu = std::min<long long>(wg_per_cu, (long long)(kLdsPerCu / lds));
    return (long long)cu_count() * wg_per_cu * 4;
  };
  int ks = 1;
  for (int cand : {4, 2}) {
    if (pairs * cand <= resident_waves(cand)) {
      ks = cand;
      break;
    }
  }
  a.ksplit = ks;
  const int per_wg = 4 / ks;
  dim3 grid((unsigned)(pairs_per_group / per_wg), (unsigned)(a.compact ? active_groups : G));
  const unsigned lds = (unsigned)lds_bytes(ks);
  if (use_lds) {
    if (up) hipLaunchKernelGGL((ffn_decode_kernel<true, kStagesLds, true>), grid, dim3(256), lds, s, a, rows_alloc);
    else hipLaunchKernelGGL((ffn_decode_kernel<false, kStagesLds, true>), grid, dim3(256), lds, s, a, rows_alloc);
  } else {
    if (up) hipLaunchKernelGGL((ffn_decode_kernel<true, kStagesReg, false>), grid, dim3(256), lds, s, a, 16);
    else hipLaunchKernelGGL((ffn_decode_kernel<false, kStagesReg, false>), grid, dim3(256), lds, s, a, 16);
  }
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
