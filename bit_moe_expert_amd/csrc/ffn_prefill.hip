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
// Tiling. A workgroup (8 waves, two per SIMD) computes a 256-row x 256-column output
// tile of one expert over K in steps of 64; each wave owns 128 x 64 of it as 4 x 2
// blocks of 32x32x16 MFMAs (on gfx950 this shape runs near the BF16 peak, while
// 16x16x32 tops out near half of it). Two waves per SIMD let one wave's MFMAs run while
// the other waits on LDS or does its share of the dequantisation (with one wave of
// 128 x 128 per SIMD the same tile ran slower). For the up projection the 256 weight
// rows are 128 gate rows and the matching 128 up rows, and each wave takes 32 of each,
// so gate and up accumulators of the same h columns sit in the same lanes and SwiGLU
// is applied in registers. An expert's last tile, when it has at most 192 (or 128)
// rows, is computed by all eight waves as 96 x 64 (or 64 x 64) tiles, again two waves
// per SIMD, and the activation rows past 192 (or 128) are neither loaded nor stored.
//
// Pipeline. Activation rows (gathered through perm_src for the up projection) and
// weight half-tiles (tiled layout: 512 contiguous bytes per 16-row block; canonical:
// 16 rows of 32 bytes) are loaded
// into one of two register sets two steps ahead of use; during step i's MFMAs, step
// i+1's set is dequantised (code * E4M3 scale is exact in BF16) and written to the
// other LDS buffer part by part, each part's registers then refilled with step i+3.
// The weights are read through the caches: every M-tile of an expert reads the same
// weight tiles, and the tile order keeps those workgroups on one XCD. One barrier
// per step. Each 16-wide K substep reads its operand fragments from LDS while
// the previous one's MFMAs run. LDS rows are XOR-swizzled in 16-byte chunks so that
// both the MFMA operand reads and the stores spread over the banks.
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
constexpr int kThreads = 512;
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
};

// LDS tiles are [rows][64] BF16, 128 bytes a row; the 16-byte chunk c of row r is stored
// at chunk c ^ swz_key(r). The key keeps both access shapes free of bank conflicts (as
// measured on gfx950): a 128-bit read serves 16 lanes at a time over 256 bytes of banks,
// i.e. two rows, so the keys of the 8 even (and of the 8 odd) rows of an aligned group of
// 16 must differ; a 128-bit write serves 8 lanes at a time over 128 bytes, so the weight
// stores (8 lanes = 8 consecutive rows, same chunk) need 8 different keys on aligned
// groups of 8 rows. The key depends only on r % 16.
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// kDense: one group of T rows, row r = token r (the shared expert); else the routed
// groups of the plan. (Separate instantiations, so that a kernel trace lists the
// routed and the shared launches apart.) kTiled: the weights' layout (tiled, else
// canonical); a compile-time choice, so the tiled form's addressing stays shifts.
template <bool kUp, bool kDense, bool kTiled>
__global__ __launch_bounds__(kThreads, 1) void ffn_prefill_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][BN * BK];
  __shared__ int sched[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

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
  if (wave == 0) {
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
  __syncthreads();
  const int g = sched[0];
  if (g < 0) return;
  const int nt = sched[3];
  const int row0 = sched[1], rows = sched[2];

  const int K = a.K, NS = K / 128, NB = a.N / 16, nsteps = K / BK;
  const float ts = a.tscale[g];

  // ---- global -> register loads ----
  // A: thread t loads rows t/8 + 64i (i = 0..3), 16-byte chunk t%8 of the step. Rows
  // past the tile's end read the tile's first row instead: their results are never
  // stored, so they need no masking.
  const int a_chunk = tid & 7;
  const uint16_t* a_src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (tid >> 3) + 64 * i;
    int src = row0 + (rr < rows ? rr : 0);
    if (kUp && !kDense) src = a.perm_src[src] / a.k;
    a_src[i] = a.act + (size_t)src * K + a_chunk * 8;
  }
  // B: unit u = tid: 16-row block u/32, lane-in-half-tile u%32 (row rn = u%16 of the
  // block, columns 32kq'..32kq'+31 of each 64-column step, kq' = (u%32)/16). Both
  // layouts keep a block's codes (16 * K/2 bytes) and scales (16 * K/16) in one range
  // at the same place; step st's 16 code bytes and 2 scale bytes of the unit sit at
  // st * step + unit offset: tiled, 512 + 64 bytes a step (half a 16 x 128 tile) in
  // lane order; canonical, 32 code bytes and 4 scale bytes a step along row rn.
  const uint8_t* b_code[1];
  const uint8_t* b_scale[1];
  int b_st[1];  // LDS element offset of the unit's row (its 4 chunks are 4*kq' + j)
  constexpr int bc_step = kTiled ? 512 : 32, bs_step = kTiled ? 64 : 4;
#pragma unroll
  for (int h = 0; h < 1; ++h) {
    const int u = tid;
    const int blk = u >> 5, l = u & 31;
    int wblk;  // weight row-block of this LDS block
    if (kUp) wblk = blk < 8 ? (nt * 128) / 16 + blk : (a.I + nt * 128) / 16 + (blk - 8);
    else wblk = (nt * BN) / 16 + blk;
    const size_t tile = ((size_t)g * NB + wblk) * NS;
    const int rn = l & 15, kq = l >> 4;
    b_code[h] = a.tcodes + tile * 1024 + (kTiled ? l * 16 : rn * (K / 2) + kq * 16);
    b_scale[h] = a.tscales + tile * 128 + (kTiled ? l * 2 : rn * (K / 16) + kq * 2);
    b_st[h] = blk * 16 + (l & 15);
  }
  const int b_kq = (tid & 31) >> 4;  // same for both units
  // LDS swizzle (swz_key): for every row a lane touches, the key depends only on the
  // lane (row offsets are multiples of 16), so the addresses are a
  // per-lane base plus immediate offsets.
  const int a_sw = swz_key(tid >> 3);
  const int a_st = (tid >> 3) * BK + ((a_chunk ^ a_sw) << 3);  // + 64*i*BK for row group i
  const int b_sw = swz_key(tid & 15);

  // Two register sets, used by alternate steps: step s's data is loaded during step
  // s - 2 and written to LDS during step s - 1, so every load has a whole step and more
  // to arrive.
  u32x4 ra[2][4], rb[2];
  uint32_t rs[2];
  // Part q of step st's global loads into set S: activation row q of this thread and,
  // for q = 3, the weight unit (whose four store parts have then all been written).
  // (groups: the activation row groups of 64 the tile needs, 4, 3 or 2)
  auto load_part = [&](auto SET, int st, int q, int groups) {
    constexpr int S = decltype(SET)::value;
    const int k0 = st * BK;
    if (q < groups) ra[S][q] = *reinterpret_cast<const u32x4*>(a_src[q] + k0);
    if (q == 3) {
      // (tiled: st * 512 and st * 64, written per 1 KB tile and half, which the
      // compiler turns into fewer live registers than the product)
      const size_t toff = kTiled ? (size_t)(st >> 1) * 1024 + (st & 1) * 512 : (size_t)st * bc_step;
      const size_t soff = kTiled ? (size_t)(st >> 1) * 128 + (st & 1) * 64 : (size_t)st * bs_step;
      rb[S] = *reinterpret_cast<const u32x4*>(b_code[0] + toff);
      rs[S] = *reinterpret_cast<const uint16_t*>(b_scale[0] + soff);
    }
  };
  // Part q (0..3) of writing set S into LDS buffer `buf`: activation row q of this
  // thread, and BF16 chunk q of the weight unit (dequantised here).
  auto store_part = [&](auto SET, int buf, int q, int groups) {
    constexpr int S = decltype(SET)::value;
    if (q < groups) *reinterpret_cast<u32x4*>(&lds_a[buf][a_st + 64 * q * BK]) = ra[S][q];
    const float sc = q < 2 ? e4m3_to_f32<0>(rs[S]) : e4m3_to_f32<1>(rs[S]);
    *reinterpret_cast<u32x4*>(&lds_b[buf][b_st[0] * BK + (((4 * b_kq + q) ^ b_sw) << 3)]) = dequant8(rb[S][q], sc);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // ---- per-wave tile: 128 rows x 64 LDS B rows as 4 x 2 blocks of 32x32x16 MFMAs ----
  // An expert's last tile of at most 192 rows (three-quarter) or 128 rows (half) is
  // computed by all eight waves as 96- or 64-row x 64 tiles (3 x 2 or 2 x 2 blocks),
  // two waves per SIMD as in a full tile; the activation rows past 192 or 128 are
  // neither loaded nor stored. Each output is the same chain of MFMAs over K in every
  // tile shape, so the shape does not change any bits.
  const int wm = wave >> 2, wn = wave & 3;
  const int r32 = lane & 31, kh = lane >> 5;  // operand row within a 32-block; K half (8 values)
  // LDS B rows of block j: up = gate rows 64wn + 32j (j < 2) then up rows
  // 128 + 64wn + 32(j-2); down = rows 128wn + 32j. Row offsets are multiples of 32.
  int boff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) boff[j] = kUp ? 128 * j + 32 * wn : 64 * wn + 32 * j;
  const int f_sw = swz_key(r32);
  const int fb_base = r32 * BK;

  auto compute = [&](auto MIC) {
    constexpr int MI = decltype(MIC)::value;  // 32-row blocks of a wave's tile: 4, 3 or 2
    // Prologue: step 0 into LDS buffer 0, steps 1 and 2 into register sets 1 and 0.
#pragma unroll
    for (int q = 0; q < 4; ++q) load_part(S0{}, 0, q, MI);
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(S0{}, 0, q, MI);
#pragma unroll
    for (int q = 0; q < 4; ++q) load_part(S1{}, min(1, nsteps - 1), q, MI);
#pragma unroll
    for (int q = 0; q < 4; ++q) load_part(S0{}, min(2, nsteps - 1), q, MI);
    __syncthreads();
    constexpr int WR = 32 * MI;        // rows of a wave's tile
    const int fa_base = (WR * wm + r32) * BK;
    f32x16 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // operand fragments of one 16-wide K substep
    u32x4 fa[MI], fb[2], na[MI], nb[2];
    auto read_frags = [&](int buf, int ks, u32x4* A, u32x4* Bv) {
      const int cs = ((2 * ks + kh) ^ f_sw) << 3;
#pragma unroll
      for (int j = 0; j < 2; ++j) Bv[j] = *reinterpret_cast<const u32x4*>(&lds_b[buf][fb_base + boff[j] * BK + cs]);
#pragma unroll
      for (int i = 0; i < MI; ++i) A[i] = *reinterpret_cast<const u32x4*>(&lds_a[buf][fa_base + 32 * i * BK + cs]);
    };
    read_frags(0, 0, fa, fb);
    // Steps come in pairs (K is a multiple of 128): step st writes set (st + 1) % 2.
    auto step = [&](auto SET, int st) {
      const int buf = st & 1;
      const int next3 = min(st + 3, nsteps - 1);  // the last steps reload themselves (never read)
      // Four 16-wide substeps. In each, the next substep's fragments are read while this
      // one's MFMAs run; then one part of step st+1 is written to the other buffer, and
      // its registers are refilled with step st+3.
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        if (ks + 1 < BK / 16) read_frags(buf, ks + 1, na, nb);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(fa[i], fb[j], acc[i][j]);
        store_part(SET, buf ^ 1, ks, MI);
        load_part(SET, next3, ks, MI);
        if (ks + 1 < BK / 16) {
#pragma unroll
          for (int i = 0; i < MI; ++i) fa[i] = na[i];
#pragma unroll
          for (int j = 0; j < 2; ++j) fb[j] = nb[j];
        }
      }
      __syncthreads();
      read_frags(buf ^ 1, 0, fa, fb);
    };
    for (int st = 0; st < nsteps; st += 2) {
      step(S1{}, st);
      step(S0{}, st + 1);
    }

    // ---- epilogue: acc[i][j][r] is row 8(r/4) + 4kh + r%4, column r32 of block (i, j) ----
    // The wave's outputs go through LDS (the operand buffers are free once every wave
    // has passed the barrier), so that each lane writes whole 16-byte row pieces: 8 (up)
    // or 16 (down) stores a wave instead of 64 or 128 of 2 bytes. A wave's LDS region is
    // its own [WR][W] BF16 block (W = 32 h columns for up, 64 y columns for down).
    __syncthreads();
    constexpr int W = kUp ? 32 : 64;
    uint16_t* stage = (wave < 4 ? &lds_a[0][0] : &lds_b[0][0]) + (wave & 3) * (128 * W);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
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
    constexpr int kPieces = WR * W / 8;  // 16-byte pieces of the wave's block
    const size_t ld = kUp ? a.I : a.N;
    const int col0 = kUp ? nt * 128 + 32 * wn : nt * BN + 64 * wn;
#pragma unroll
    for (int c = 0; c < kPieces / 64; ++c) {
      const int piece = 64 * c + lane, lr = piece / (W / 8), lc = (piece % (W / 8)) * 8;
      const int tr = WR * wm + lr;
      if (tr < rows)
        *reinterpret_cast<u32x4*>(a.out + (size_t)(row0 + tr) * ld + col0 + lc) =
            *reinterpret_cast<const u32x4*>(stage + lr * W + lc);
    }
  };
  if (rows <= BM / 2) compute(std::integral_constant<int, 2>{});
  else if (rows <= kTq) compute(std::integral_constant<int, 3>{});
  else compute(std::integral_constant<int, 4>{});
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
             w13.tiled ? 1 : 0};
  return launch(true, a, m_tile_bound(offsets, T, k, G), s);
}

hipError_t launch_ffn_down_prefill(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H,
                                   int I, W4View w2, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  GemmArgs a{h, offsets, nullptr, 1, T, w2.packed, w2.scales, w2.tscale, H, I, I, G, y, 0, 0,
             w2.tiled ? 1 : 0};
  return launch(false, a, m_tile_bound(offsets, T, k, G), s);
}

}  // namespace moe4
