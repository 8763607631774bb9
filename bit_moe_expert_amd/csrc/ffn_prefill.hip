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
// SwiGLU is applied in registers. A tile of fewer rows (an expert's last) is computed
// as MI x 2 blocks a wave, MI = its rows rounded up to 32 (2 to 8), and the activation
// rows past 32 MI are neither loaded nor computed.
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
#include "prefill_common.hpp"

namespace moe4 {

namespace {

using namespace prefill;

constexpr int kBWave = 2 * 1024 + 2 * 256;  // weight bytes one wave copies per K step

// 32x32x16 FP16 MFMA (operands in the lanes and slots of the BF16 one)
__device__ __forceinline__ f32x16 mfma32x32x16_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// One wave's weight operands of a K step, read from its LDS slot: the 16 code bytes
// of each of its two 32-row blocks and the dword holding their two E4M3 scales.
struct WRaw {
  u32x4 c[2];
  uint32_t s[2];
};

// kDense: one group of T rows, row r = token r (the shared expert); else the routed
// groups of the plan. (Separate instantiations, so that a kernel trace lists the
// routed and the shared launches apart.) kTiled: the weights' layout (tiled, else
// canonical); a compile-time choice, so the tiled form's addressing stays shifts.
// kF16 (up only): the activations are FP16 rows scaled by a power of two each (act =
// x * 2^-xexp[token]); the weights are dequantised into FP16 (two instructions per
// pair of weights instead of four) and multiplied by FP16 MFMAs, and the epilogue
// scales each row's FP32 sums back by 2^xexp. Every product is exact in both forms and
// a power-of-two scale scales every FP32 partial sum exactly, so h has the BF16 form's
// bits while the row's values are exact in FP16.
template <bool kUp, bool kDense, bool kTiled, bool kF16>
__device__ __forceinline__ void prefill_gemm(const GemmArgs& a) {
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
  // kF16: the tile's per-row exponents (row r's token's xexp), copied in at the start
  __shared__ __attribute__((aligned(16))) int32_t rexp[kF16 ? BM : 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (wave == 0) tile_schedule<kDense>(a, lane, sched);
  __syncthreads();
  const int g = sched[0];
  if (g < 0) return;
  const int nt = sched[3];
  const int row0 = sched[1], rows = sched[2];
  // the token of tile row tid (rows past the tile's end take its first row)
  int rexp_tok = 0;
  if constexpr (kF16) {
    rexp_tok = row0 + (tid < rows ? tid : 0);
    if (!kDense) rexp_tok = a.perm_src[rexp_tok] / a.k;
  }

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
    constexpr int MI = decltype(MIC)::value;  // 32-row blocks of the tile: 2 to 8
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
        if constexpr (kF16) {
          const f16x2 sc2 = e4m3x2_to_f16(r.s[j]);
          Bv[j] = dequant8_f16(r.c[j][s], s < 2 ? sc2[0] : sc2[1]);
        } else {
          const float sc = s < 2 ? e4m3_to_f32<0>(r.s[j]) : e4m3_to_f32<1>(r.s[j]);
          Bv[j] = dequant8(r.c[j][s], sc);
        }
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
    // kF16: the row exponents, one 4-byte copy per thread (issued after the first two
    // steps' copies, so the waits below count them as part of step 1; they have landed
    // by the epilogue's wait for everything)
    if constexpr (kF16)
      __builtin_amdgcn_global_load_lds(a.xexp + rexp_tok, (__attribute__((address_space(3))) void*)&rexp[64 * wv], 4,
                                       0, 0);
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
          for (int j = 0; j < 2; ++j) {
            if constexpr (kF16) acc[i][j] = mfma32x32x16_f16(fa[i], fb[j], acc[i][j]);
            else acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
          }
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
          __builtin_amdgcn_sched_group_barrier(0x100, 4 + (MI & 1), 0);
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
      for (int r = 0; r < 16; r += 2) {
        // rows lr and lr + 1 of column r32: one packed conversion, two 16-bit stores
        const int lr = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        if constexpr (kF16) {
          // this row pair's exponents (rows lr, lr + 1 of the tile)
          const int e0 = rexp[lr], e1 = rexp[lr + 1];
          const uint32_t p = pack_bf16x2(
              silu_mul(__builtin_ldexpf(ts * acc[i][0][r], e0), __builtin_ldexpf(ts * acc[i][1][r], e0)),
              silu_mul(__builtin_ldexpf(ts * acc[i][0][r + 1], e1), __builtin_ldexpf(ts * acc[i][1][r + 1], e1)));
          stage[lr * W + r32] = (uint16_t)p;
          stage[(lr + 1) * W + r32] = (uint16_t)(p >> 16);
        } else if (kUp) {
          const uint32_t p = pack_bf16x2(silu_mul(ts * acc[i][0][r], ts * acc[i][1][r]),
                                         silu_mul(ts * acc[i][0][r + 1], ts * acc[i][1][r + 1]));
          stage[lr * W + r32] = (uint16_t)p;
          stage[(lr + 1) * W + r32] = (uint16_t)(p >> 16);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t p = pack_bf16x2(ts * acc[i][j][r], ts * acc[i][j][r + 1]);
            stage[lr * W + 32 * j + r32] = (uint16_t)p;
            stage[(lr + 1) * W + 32 * j + r32] = (uint16_t)(p >> 16);
          }
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
  // 32-row blocks a wave computes: the tile's rows rounded up to 32, from 2 to 8 (only
  // the copies and MFMAs of those rows run; the weights are loaded whole whatever MI)
  if (rows <= 64) compute(std::integral_constant<int, 2>{});
  else if (rows <= 96) compute(std::integral_constant<int, 3>{});
  else if (rows <= 128) compute(std::integral_constant<int, 4>{});
  else if (rows <= 160) compute(std::integral_constant<int, 5>{});
  else if (rows <= 192) compute(std::integral_constant<int, 6>{});
  else if (rows <= 224) compute(std::integral_constant<int, 7>{});
  else compute(std::integral_constant<int, 8>{});
}

template <bool kUp, bool kDense, bool kTiled>
__global__ __launch_bounds__(kThreads, 1) void ffn_prefill_kernel(GemmArgs a) {
  prefill_gemm<kUp, kDense, kTiled, false>(a);
}
// the FP16-activation form of the up projection (its own name in kernel traces)
template <bool kDense, bool kTiled>
__global__ __launch_bounds__(kThreads, 1) void ffn_prefill_f16_kernel(GemmArgs a) {
  prefill_gemm<true, kDense, kTiled, true>(a);
}

hipError_t launch(bool up, GemmArgs a, long long m_tiles, hipStream_t s) {
  const dim3 g = size_grid(a, up, m_tiles), b(kThreads);
  const bool dense = a.offsets == nullptr;
  if (a.xexp) {
    if (!up) return hipErrorInvalidValue;
    if (a.tiled) {
      if (!dense) hipLaunchKernelGGL((ffn_prefill_f16_kernel<false, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((ffn_prefill_f16_kernel<true, true>), g, b, 0, s, a);
    } else {
      if (!dense) hipLaunchKernelGGL((ffn_prefill_f16_kernel<false, false>), g, b, 0, s, a);
      else hipLaunchKernelGGL((ffn_prefill_f16_kernel<true, false>), g, b, 0, s, a);
    }
    return hipGetLastError();
  }
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


}  // namespace

bool prefill_shape_ok(int H, int I) { return H % BN == 0 && I % 128 == 0; }

hipError_t launch_ffn_up_prefill(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                                 int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{x, offsets, perm_src, k, T, w13.packed, w13.scales, w13.tscale, 2 * I, H, I, G, h, 0, 0,
             w13.tiled ? 1 : 0, nullptr, nullptr, nullptr, nullptr};
  return launch(true, a, m_tile_bound(offsets, T, k, G), s);
}

hipError_t launch_ffn_up_prefill_f16(const uint16_t* x16, const int32_t* xexp, const int32_t* offsets,
                                     const int32_t* perm_src, int k, int T, int G, int H, int I, W4View w13,
                                     uint16_t* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{x16, offsets, perm_src, k, T, w13.packed, w13.scales, w13.tscale, 2 * I, H, I, G, h, 0, 0,
             w13.tiled ? 1 : 0, nullptr, nullptr, nullptr, nullptr, xexp};
  return launch(true, a, m_tile_bound(offsets, T, k, G), s);
}

hipError_t launch_ffn_down_prefill(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H,
                                   int I, W4View w2, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{h, offsets, nullptr, 1, T, w2.packed, w2.scales, w2.tscale, H, I, I, G, y, 0, 0,
             w2.tiled ? 1 : 0, nullptr, nullptr, nullptr, nullptr};
  return launch(false, a, m_tile_bound(offsets, T, k, G), s);
}

}  // namespace moe4
