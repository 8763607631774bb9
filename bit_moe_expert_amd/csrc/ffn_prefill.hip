// Grouped W4A16 expert FFN for many rows per expert (prefill): an MFMA grouped GEMM.
//
// Prefill pushes all prompt tokens through one large matmul and is bound by the
// matrix units, not by memory (the GB10 bandwidth budget article, section
// "Mechanism: decode is bandwidth-bound, prefill is compute-bound"); the weights
// are NVFP4 computed against BF16 activations, i.e. W4A16 (bear-blog article on
// TensorFold 1.0.12 / PR804, section "NVFP4 is neither uniform 4-bit nor all-FP4
// compute"). So the 4-bit weights are dequantised exactly into BF16 once per
// workgroup tile and fed to BF16 MFMAs with FP32 accumulation.
//
// Tiling. A workgroup of 4 waves (one per SIMD) computes a 256-row x 256-column output
// tile of one expert over K in steps of 64; each wave owns all 256 rows of 64 columns
// as 8 x 2 blocks of 32x32x16 MFMAs (on gfx950 this shape runs near the BF16 peak,
// while 16x16x32 tops out near half of it), with its 256 accumulators in the AGPRs.
// Because a wave owns its 64 weight rows alone, each weight is read and dequantised
// once per tile, by one wave, straight into its MFMA operand registers: the weights
// never pass through a shared LDS tile. Only the activations are shared: each wave
// reads every activation row from LDS, 32 KB a step for 64 x 16 x 256 x 2 MFMA flops,
// half the LDS bytes per flop of 128 x 64 wave tiles that take both operands from LDS.
// For the up projection the 64 weight rows are 32 gate rows and the matching 32 up
// rows, so gate and up accumulators of the same h columns sit in the same lanes and
// SwiGLU is applied in registers. An expert's last tile, when it has at most 192 (or
// 128) rows, is computed as 6 x 2 (or 4 x 2) blocks a wave, and the activation rows
// past 192 (or 128) are neither loaded nor computed.
//
// Pipeline. Every load is a direct-to-LDS copy (global_load_lds), issued two K steps
// ahead into a ring of three LDS slots: the activation rows of the tile (gathered
// through perm_src for the up projection), 8 rows per instruction, and each wave's own
// weight codes and scales (tiled layout: 512 contiguous bytes per 16-row block and
// step; canonical: 16 rows of 32 bytes). With only such copies in flight the wait at
// the top of a step can leave the next step's copies outstanding (s_waitcnt with a
// count), then one barrier makes the step's slot visible and frees the slot read two
// steps ago. Within a step each 16-wide K substep reads its activation fragments from
// LDS and dequantises its weight fragments (code * E4M3 scale is exact in BF16) while
// the previous substep's MFMAs run. LDS rows are XOR-swizzled in 16-byte chunks (the
// copies place a row's chunks at swizzled positions) so that the fragment reads of 16
// rows at a time spread over all banks.
//
// Scheduling. One grid covers (expert M-tile, N-tile) pairs up to a bound; each
// workgroup counts the per-expert tiles from the offsets, which gives the number of
// real tiles and its own expert. The real tiles are dealt to the 8 XCDs (workgroup
// ids go round-robin to them) in equal contiguous runs with N fastest: the workgroups
// sharing an activation tile, and an expert's weights, meet in the same L2, and every
// XCD gets the same share of work. (Dealing the bound's range instead left the last
// XCDs with only empty tiles: at prefill about a sixth of the CUs idled.)
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kTq = 192;  // rows of a three-quarter tile
constexpr int kThreads = 256;
constexpr int kBWave = 2 * 1024 + 2 * 256;  // weight bytes one wave copies per K step
constexpr int kXcds = 8;
constexpr int kMaxExperts = 256;  // the ABI's bound on G

struct GemmArgs {
  const uint16_t* act;      // up: x [T][H]; down: h [R][I]
  const int32_t* offsets;   // [G+1] or NULL (dense: one group of T rows)
  const int32_t* perm_src;  // up only: row -> flat pair (token = pair / k); NULL = identity
  int k;
  int T;
  const uint8_t* tcodes;
  const uint8_t* tscales;
  const float* tscale;
  int N, K, I;              // up: N = 2I, K = H; down: N = H, K = I
  int G;
  uint16_t* out;            // up: h [R][I]; down: y [R][N]
  int n_tiles;              // output column tiles per expert
  int total;                // grid size (multiple of kXcds)
  int tiled;                // weights in the tiled layout, else canonical
  // FP8 (W4A8) form only:
  const uint8_t* act8;      // E4M3 activations [rows][K] (up: x8 [T][H]; down: h8 [R][I])
  const uint8_t* ascale;    // their E8M0 block scales [rows][K/32]
  uint8_t* out8;            // up: h8 [R][I] out
  uint8_t* oscale;          // up: h8's block scales [R][I/32] out
};

// One wave's weight operands of a K step, read from its LDS slot: the 16 code bytes
// of each of its two 32-row blocks and the dword holding their two E4M3 scales.
struct WRaw {
  u32x4 c[2];
  uint32_t s[2];
};

// LDS tiles are [rows][64] BF16, 128 bytes a row; the 16-byte chunk c of row r is stored
// at chunk c ^ swz_key(r). The key keeps both access shapes free of bank conflicts (as
// measured on gfx950): a 128-bit read serves 16 lanes at a time over 256 bytes of banks,
// i.e. two rows, so the keys of the 8 even (and of the 8 odd) rows of an aligned group of
// 16 must differ; a 128-bit write serves 8 lanes at a time over 128 bytes, so the weight
// stores (8 lanes = 8 consecutive rows, same chunk) need 8 different keys on aligned
// groups of 8 rows. The key depends only on r % 16.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Tile schedule. An expert's M-tiles are full tiles (more than 192 rows) and at most
// one shorter last tile: three-quarter (129 to 192 rows) or half (at most 128 rows,
// about two thirds the cost of a full one). Wave 0 counts the three kinds per expert
// (inclusive prefixes over the experts, 64 a round, kept in registers). The grid is
// sized from a bound; the real tiles are dealt to the 8 XCDs (workgroup ids go
// round-robin to them), each kind in equal contiguous runs with N fastest: XCD x runs
// its share of the full tiles, then of the three-quarter ones, then of the half ones.
// So the workgroups sharing an activation tile, and an
// expert's weights, meet in the same L2, every XCD gets the same amount of work
// whatever the routing, and each XCD ends on short tiles. Workgroups past their XCD's
// runs exit at once. (Dealing the bound's range in one run left the last XCDs with
// empty tiles, and XCDs with the small experts ran out early: about a fifth of the
// CU time idled at prefill.)
// Run by one wave (64 lanes); lane 0 writes {expert or -1, first row, rows, N-tile}.
template <bool kDense>
__device__ __forceinline__ void tile_schedule(const GemmArgs& a, int lane, int* sched) {
  int g = -1, r0 = 0, rows = 0, nt = 0;
  const int j = blockIdx.x / kXcds, x = blockIdx.x % kXcds;
  // tiles of each class for an expert of cnt rows
  auto classes = [](int cnt, int& f, int& t, int& h) {
    const int rem = cnt % BM;
    f = cnt / BM + (rem > kTq ? 1 : 0);
    t = rem > BM / 2 && rem <= kTq ? 1 : 0;
    h = rem != 0 && rem <= BM / 2 ? 1 : 0;
  };
  // this workgroup's place in its XCD's runs: class (0 full, 1 three-quarter, 2 half)
  // and the index of its tile within the class, or q = -1
  auto place = [&](int n_f, int n_t, int n_h, int& q, int& cls) {
    const int per_f = (n_f + kXcds - 1) / kXcds, per_t = (n_t + kXcds - 1) / kXcds;
    const int per_h = (n_h + kXcds - 1) / kXcds;
    q = -1;
    cls = 0;
    if (j < per_f) {
      q = x * per_f + j;
      if (q >= n_f) q = -1;
    } else if (j - per_f < per_t) {
      q = x * per_t + (j - per_f);
      cls = 1;
      if (q >= n_t) q = -1;
    } else if (j - per_f - per_t < per_h) {
      q = x * per_h + (j - per_f - per_t);
      cls = 2;
      if (q >= n_h) q = -1;
    }
  };
  if constexpr (!kDense) {
    int incl_f[kMaxExperts / 64], incl_t[kMaxExperts / 64], incl_h[kMaxExperts / 64];
    int first[kMaxExperts / 64], count[kMaxExperts / 64];  // expert 64c + lane's rows
    int carry_f = 0, carry_t = 0, carry_h = 0;
#pragma unroll
    for (int c = 0; c < kMaxExperts / 64; ++c) {
      const int e = 64 * c + lane;
      first[c] = e < a.G ? a.offsets[e] : 0;
      const int cnt = e < a.G ? a.offsets[e + 1] - first[c] : 0;
      count[c] = cnt;
      int f, t, h;
      classes(cnt, f, t, h);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int of = __shfl_up(f, off), ot = __shfl_up(t, off), oh = __shfl_up(h, off);
        if (lane >= off) {
          f += of;
          t += ot;
          h += oh;
        }
      }
      incl_f[c] = carry_f + f;
      incl_t[c] = carry_t + t;
      incl_h[c] = carry_h + h;
      carry_f += __shfl(f, 63);
      carry_t += __shfl(t, 63);
      carry_h += __shfl(h, 63);
    }
    int q, cls;
    place(carry_f * a.n_tiles, carry_t * a.n_tiles, carry_h * a.n_tiles, q, cls);
    if (q >= 0) {
      const int m = q / a.n_tiles;
      nt = q % a.n_tiles;
      auto incl_of = [&](int c) { return cls == 0 ? incl_f[c] : (cls == 1 ? incl_t[c] : incl_h[c]); };
#pragma unroll
      for (int c = 0; c < kMaxExperts / 64; ++c) {
        const int e = 64 * c + lane;
        const int incl = incl_of(c);
        const int prev = __shfl_up(incl, 1);  // every lane takes part in both shuffles
        const int before = c == 0 ? 0 : __shfl(incl_of(c > 0 ? c - 1 : 0), 63);
        const int excl = lane == 0 ? before : prev;
        const uint64_t hit = __ballot(e < a.G && m >= excl && m < incl);
        if (hit && g < 0) {
          const int src = __ffsll((long long)hit) - 1;
          g = __shfl(e, src);
          const int mt = cls ? 0 : m - __shfl(excl, src);
          r0 = __shfl(first[c], src);  // from the counting loads, not a second round trip
          const int cnt = __shfl(count[c], src);
          // a three-quarter or half tile is the expert's last M-tile
          const int m0 = cls ? cnt / BM : mt;
          r0 += m0 * BM;
          rows = min(BM, cnt - m0 * BM);
        }
      }
    }
  } else {
    // dense: one group of T rows
    const int cnt = a.T;
    int f, t, h, q, cls;
    classes(cnt, f, t, h);
    place(f * a.n_tiles, t * a.n_tiles, h * a.n_tiles, q, cls);
    if (q >= 0) {
      g = 0;
      nt = q % a.n_tiles;
      const int m0 = cls ? cnt / BM : q / a.n_tiles;
      r0 = m0 * BM;
      rows = min(BM, cnt - m0 * BM);
    }
  }
  if (lane == 0) {
    sched[0] = g;
    sched[1] = r0;  // first row of the tile
    sched[2] = rows;
    sched[3] = nt;
  }
}

// kDense: one group of T rows, row r = token r (the shared expert); else the routed
// groups of the plan. (Separate instantiations, so that a kernel trace lists the
// routed and the shared launches apart.) kTiled: the weights' layout (tiled, else
// canonical); a compile-time choice, so the tiled form's addressing stays shifts.
template <bool kUp, bool kDense, bool kTiled>
__global__ __launch_bounds__(kThreads, 1) void ffn_prefill_kernel(GemmArgs a) {
  // three activation buffers [256][64] BF16 (the ring of steps st, st+1, st+2) and a
  // fourth one for the epilogue's staging; separate arrays, so that the compiler can
  // tell a direct-to-LDS copy into one from reads of another
  __shared__ __attribute__((aligned(16))) uint16_t lds0[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t lds1[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t lds2[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t lds3[BM * BK];
  // weight ring: per slot and wave, two blocks' code bytes (1 KB each, lane order) and
  // their scale dwords (256 B each)
  __shared__ __attribute__((aligned(16))) uint8_t ldsb0[4 * kBWave];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb1[4 * kBWave];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb2[4 * kBWave];
  __shared__ int sched[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (wave == 0) tile_schedule<kDense>(a, lane, sched);
  __syncthreads();
  const int g = sched[0];
  if (g < 0) return;
  const int nt = sched[3];
  const int row0 = sched[1], rows = sched[2];

  const int K = a.K, NS = K / 128, NB = a.N / 16, nsteps = K / BK;
  const float ts = a.tscale[g];
  const int r32 = lane & 31, hh = lane >> 5;  // MFMA operand row / column; K half
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // ---- weights: this wave's 64 B rows, straight from memory into registers ----
  // Block j (0, 1) is 32 weight rows: up = gate rows 128nt + 32w .. +31 (j = 0) and the
  // matching up rows (j = 1), so gate and up accumulators of one h column sit in the
  // same lane; down = rows 256nt + 64w + 32j .. +31. In a K step (64 columns) lane l
  // takes row l%32 of the block and the 32 columns 32hh .. 32hh+31 of the step: 16 code
  // bytes and the 2 scale bytes of those columns. (The MFMA only needs A and B to agree
  // on which K each lane group and slot stands for: in substep s lane group hh takes
  // K = 32hh + 8s .. +7 of the step, in A as well.)
  const uint8_t* bcode[2];
  const uint8_t* bscale[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n0 = kUp ? (j == 0 ? nt * 128 + 32 * wv : a.I + nt * 128 + 32 * wv) : nt * BN + 64 * wv + 32 * j;
    const int row = n0 + r32;
    if constexpr (kTiled) {
      // tile (g, row/16, kt): lane rn + 16 kq of it, kq = 2 (st % 2) + hh
      const size_t tile = ((size_t)g * NB + row / 16) * NS;
      bcode[j] = a.tcodes + tile * 1024 + ((row & 15) + 16 * hh) * 16;
      bscale[j] = a.tscales + tile * 128 + ((row & 15) + 16 * hh) * 2;
    } else {
      const size_t r = (size_t)g * a.N + row;
      bcode[j] = a.tcodes + r * (K / 2) + hh * 16;
      bscale[j] = a.tscales + r * (K / 16) + hh * 2;
    }
  }

  auto compute = [&](auto MIC) {
    constexpr int MI = decltype(MIC)::value;  // 32-row blocks of the tile: 8, 6 or 4
    constexpr int RW = 8 * MI;                // activation rows each wave copies
    // ---- activations: rows of the tile straight into LDS (global_load_lds) ----
    // Wave w copies LDS rows RW*w .. RW*w + RW-1, 8 rows (1 KB) per instruction: lane l
    // fills row RW*w + 8i + l/8, 16-byte position l%8, with the row's global chunk
    // (l%8) ^ swz_key(row), so that chunk c of row r sits at position c ^ swz_key(r).
    // Rows past the tile's end copy its first row: their results are never stored.
    // (sized 8, the most MI, rather than MI: passing an element of an array sized by
    // the lambda's template value to the copy builtin made hipcc's host pass drop the
    // kernel's launch stubs)
    const uint16_t* asrc[8];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int rr = RW * wv + 8 * i + (lane >> 3);
      int src = row0 + (rr < rows ? rr : 0);
      if (kUp && !kDense) src = a.perm_src[src] / a.k;
      asrc[i] = a.act + (size_t)src * K + (((lane & 7) ^ swz_key(rr)) << 3);
    }
    auto buf_of = [&](auto RC) -> uint16_t* {
      constexpr int R = decltype(RC)::value;
      return R == 0 ? lds0 : (R == 1 ? lds1 : lds2);
    };
    auto load_a = [&](int st, uint16_t* b) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
        __builtin_amdgcn_global_load_lds(asrc[i] + st * BK,
                                         (__attribute__((address_space(3))) void*)&b[(RW * wv + 8 * i) * BK],
                                         16, 0, 0);
    };
    // weights: also straight into LDS (this wave's own region of the slot), so that
    // every load in flight is a direct-to-LDS copy and the waits on them can be counted
    auto bbuf_of = [&](auto RC) -> uint8_t* {
      constexpr int R = decltype(RC)::value;
      return (R == 0 ? ldsb0 : (R == 1 ? ldsb1 : ldsb2)) + wv * kBWave;
    };
    auto load_b = [&](int st, uint8_t* b) {
      // step st's offsets from the bases (tiled: 1 KB + 128 B per 128-column tile, half
      // of it per step; canonical: 32 + 4 bytes per step along the row)
      const size_t co = kTiled ? (size_t)(st >> 1) * 1024 + (st & 1) * 512 : (size_t)st * 32;
      const size_t so = kTiled ? (size_t)(st >> 1) * 128 + (st & 1) * 64 : (size_t)st * 4;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint8_t* cp = bcode[j] + co;
        // the dword holding this lane's 2 scale bytes
        const uint8_t* sp = bscale[j] + so;
        const uint8_t* sd = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(sp) & ~uintptr_t(3));
        __builtin_amdgcn_global_load_lds(cp, (__attribute__((address_space(3))) void*)(b + j * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(sd, (__attribute__((address_space(3))) void*)(b + 2048 + j * 256), 4, 0, 0);
      }
    };
    // this lane's two 16-bit scale pairs sit in the upper or lower half of its dword
    const int sc_shift = (int)((reinterpret_cast<uintptr_t>(bscale[0]) & 2) * 8);
    f32x16 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int key = swz_key(r32);
    auto read_a = [&](auto RC, int s, u32x4* A) {
      const uint16_t* b = buf_of(RC);
      const int cs = ((4 * hh + s) ^ key) << 3;
#pragma unroll
      for (int i = 0; i < MI; ++i) A[i] = *reinterpret_cast<const u32x4*>(&b[(32 * i + r32) * BK + cs]);
    };
    auto read_b = [&](auto RC, WRaw& r) {
      const uint8_t* b = bbuf_of(RC);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        r.c[j] = *reinterpret_cast<const u32x4*>(b + j * 1024 + lane * 16);
        r.s[j] = *reinterpret_cast<const uint32_t*>(b + 2048 + j * 256 + lane * 4) >> sc_shift;
      }
    };
    auto deq_b = [&](const WRaw& r, int s, u32x4* Bv) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float sc = s < 2 ? e4m3_to_f32<0>(r.s[j]) : e4m3_to_f32<1>(r.s[j]);
        Bv[j] = dequant8(r.c[j][s], sc);
      }
    };
    // s_waitcnt vmcnt(MI + 4) lgkmcnt(0): at most one step's copies (MI activation
    // copies, 4 weight copies) still in flight, every LDS read of this wave done
    // (gfx9 encoding, expcnt left at its maximum)
    constexpr int kAfter = MI + 4;
    constexpr int kWait = (kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (0 << 8);

    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    // The operands of the next MFMA substep, carried across steps: the last substep of
    // step st reads step st+1's first fragments.
    WRaw raw;
    u32x4 fa[MI], fb[2];
    // Prologue: steps 0 and 1 in flight; step 0 landed everywhere; its first operands.
    load_a(0, buf_of(C0{}));
    load_b(0, bbuf_of(C0{}));
    load_a(min(1, nsteps - 1), buf_of(C1{}));
    load_b(min(1, nsteps - 1), bbuf_of(C1{}));
    __builtin_amdgcn_s_waitcnt(kWait);
    asm volatile("s_barrier" ::: "memory");
    read_b(C0{}, raw);
    read_a(C0{}, 0, fa);
    deq_b(raw, 0, fb);
    // One K step from ring slot R (= st % 3, a compile-time index). Its substep 0
    // operands are in fa / fb. One barrier a step, before the last substep: by then
    // every wave has read all of step st but the last substep's fragments (which it
    // holds), so the slot of step st-1 is free for the copies of step st+2 issued at
    // the next step's start, and every wave's copies of step st+1 have landed, so the
    // last substep can fetch step st+1's first operands under its MFMAs. (A bare
    // s_barrier: a workgroup fence would also wait for the copies of step st+2, which
    // are in flight on purpose.)
    auto step = [&](auto RC, int st) {
      constexpr int R = decltype(RC)::value;
      constexpr int R1 = (R + 1) % 3, R2 = (R + 2) % 3;
      using CR1 = std::integral_constant<int, R1>;
      using CR2 = std::integral_constant<int, R2>;
      const int nx = min(st + 2, nsteps - 1);  // the last steps reload themselves (never read)
      u32x4 na[MI], nb[2];
      WRaw raw_next;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        if (s == BK / 16 - 1) {
          __builtin_amdgcn_s_waitcnt(kWait);
          asm volatile("s_barrier" ::: "memory");
        }
        // One wave per SIMD hides nothing by itself: the next substep's fragment reads
        // and dequantisation (and in substep 0 the copies of step st+2) are spread
        // between this substep's MFMAs, so the MFMA pipe never waits on them.
        if (s == 0) {
          load_a(nx, buf_of(CR2{}));
          load_b(nx, bbuf_of(CR2{}));
        }
        if (s + 1 < BK / 16) {
          read_a(RC, s + 1, na);
          deq_b(raw, s + 1, nb);
        } else {
          read_b(CR1{}, raw_next);
          read_a(CR1{}, 0, na);
          deq_b(raw_next, 0, nb);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
        if (s + 1 < BK / 16) {
#pragma unroll
          for (int g2 = 0; g2 < MI; ++g2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            if (s == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // VMEM (copies)
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
          }
        } else {
          // the next step's reads first (the weight bytes, whose dequantisation waits
          // for them, then the activation fragments), the dequantisation after them
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int g2 = 0; g2 < MI / 2; ++g2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
#pragma unroll
          for (int g2 = 0; g2 < 2 * MI - 1 - MI / 2; ++g2) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = na[i];
        fb[0] = nb[0];
        fb[1] = nb[1];
      }
      raw = raw_next;
    };
    // The loop body runs whole rounds of the ring, with no branch inside, so that the
    // compiler's own waits see the same loads in flight on every path; the steps past
    // the last whole round follow it.
    int st = 0;
    for (const int st_end = nsteps - nsteps % 3; st < st_end; st += 3) {
      step(C0{}, st);
      step(C1{}, st + 1);
      step(C2{}, st + 2);
    }
    if (st < nsteps) step(C0{}, st);
    if (st + 1 < nsteps) step(C1{}, st + 1);
    // every load issued has landed before the LDS is reused (the last ones are reloads)
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: acc[i][j][r] is row 32i + 8(r/4) + 4hh + r%4, column r32 of block j ----
    // The wave's outputs go through LDS (its own [256][W] BF16 region: W = 32 h columns
    // for up, 64 y columns for down) so that each lane writes whole 16-byte row pieces.
    __syncthreads();
    constexpr int W = kUp ? 32 : 64;
    // (wave w's region: the first W * 256 elements of buffer w; buffers are 256 x 64)
    uint16_t* stage = (wv == 0 ? lds0 : wv == 1 ? lds1 : wv == 2 ? lds2 : lds3);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
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
    constexpr int kPieces = 32 * MI * W / 8;  // 16-byte pieces of the wave's block
    const size_t ld = kUp ? a.I : a.N;
    const int col0 = kUp ? nt * 128 + 32 * wv : nt * BN + 64 * wv;
#pragma unroll
    for (int c = 0; c < kPieces / 64; ++c) {
      const int piece = 64 * c + lane, lr = piece / (W / 8), lc = (piece % (W / 8)) * 8;
      if (lr < rows)
        *reinterpret_cast<u32x4*>(a.out + (size_t)(row0 + lr) * ld + col0 + lc) =
            *reinterpret_cast<const u32x4*>(stage + lr * W + lc);
    }
  };
  if (rows <= BM / 2) compute(std::integral_constant<int, 4>{});
  else if (rows <= kTq) compute(std::integral_constant<int, 6>{});
  else compute(std::integral_constant<int, 8>{});
}

// ---------------------------------------------------------------------------
// The FP8 form (W4A8): activations as block-scaled E4M3 (32 values per E8M0 scale,
// quant.hip), weights dequantised and rounded to E4M3, gfx950's block-scaled
// 32x32x64 FP8 MFMA (twice the BF16 rate). The structure is the BF16 kernel's: four
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
// ---------------------------------------------------------------------------
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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (wave == 0) tile_schedule<kDense>(a, lane, sched);
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
        Bv[j] = dequant32_fp8(cs, __builtin_amdgcn_perm(ss[1], ss[0], ssel));
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
    constexpr int kHalves = kUp ? 1 : 2;  // down: 128 rows of 64 columns at a time
    constexpr int HR = 32 * MI / kHalves;   // rows per half
#pragma unroll
    for (int half = 0; half < kHalves; ++half) {
#pragma unroll
      for (int i = half * MI / kHalves; i < (half + 1) * MI / kHalves; ++i) {
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
        constexpr int kPieces = HR * W / 8;
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
  if (rows <= BM / 2) compute(std::integral_constant<int, 4>{});
  else if (rows <= kTq) compute(std::integral_constant<int, 6>{});
  else compute(std::integral_constant<int, 8>{});
}

hipError_t launch(bool up, GemmArgs a, long long m_tiles, hipStream_t s) {
  a.n_tiles = up ? a.I / 128 : a.N / BN;
  const long long tiles = m_tiles * a.n_tiles;
  // each of the three runs of an XCD (full, three-quarter, half tiles) may round up by one
  a.total = (int)((tiles + kXcds - 1) / kXcds * kXcds) + 3 * kXcds;
  const dim3 g(a.total), b(kThreads);
  const bool dense = a.offsets == nullptr;
  if (a.tiled) {
    if (!dense && up) hipLaunchKernelGGL((ffn_prefill_kernel<true, false, true>), g, b, 0, s, a);
    if (!dense && !up) hipLaunchKernelGGL((ffn_prefill_kernel<false, false, true>), g, b, 0, s, a);
    if (dense && up) hipLaunchKernelGGL((ffn_prefill_kernel<true, true, true>), g, b, 0, s, a);
    if (dense && !up) hipLaunchKernelGGL((ffn_prefill_kernel<false, true, true>), g, b, 0, s, a);
  } else {
    if (!dense && up) hipLaunchKernelGGL((ffn_prefill_kernel<true, false, false>), g, b, 0, s, a);
    if (!dense && !up) hipLaunchKernelGGL((ffn_prefill_kernel<false, false, false>), g, b, 0, s, a);
    if (dense && up) hipLaunchKernelGGL((ffn_prefill_kernel<true, true, false>), g, b, 0, s, a);
    if (dense && !up) hipLaunchKernelGGL((ffn_prefill_kernel<false, true, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_fp8(bool up, GemmArgs a, long long m_tiles, hipStream_t s) {
  a.n_tiles = up ? a.I / 128 : a.N / BN;
  const long long tiles = m_tiles * a.n_tiles;
  a.total = (int)((tiles + kXcds - 1) / kXcds * kXcds) + 3 * kXcds;
  const dim3 g(a.total), b(kThreads);
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

long long m_tile_bound(const int32_t* offsets, int T, int k, int G) {
  if (!offsets) return (T + BM - 1) / BM;
  return ((long long)T * k + BM - 1) / BM + G;  // each expert adds at most one partial tile
}

}  // namespace

bool prefill_shape_ok(int H, int I) { return H % BN == 0 && I % 128 == 0; }

hipError_t launch_ffn_up_prefill(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                                 int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{x, offsets, perm_src, k, T, w13.packed, w13.scales, w13.tscale, 2 * I, H, I, G, h, 0, 0,
             w13.tiled ? 1 : 0, nullptr, nullptr, nullptr, nullptr};
  return launch(true, a, m_tile_bound(offsets, T, k, G), s);
}

hipError_t launch_ffn_down_prefill(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H,
                                   int I, W4View w2, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{h, offsets, nullptr, 1, T, w2.packed, w2.scales, w2.tscale, H, I, I, G, y, 0, 0,
             w2.tiled ? 1 : 0, nullptr, nullptr, nullptr, nullptr};
  return launch(false, a, m_tile_bound(offsets, T, k, G), s);
}

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
