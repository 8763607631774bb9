// Shared pieces of the two prefill grouped GEMMs (the W4A16 one in ffn_prefill.hip,
// the FP8 W4A8 one in ffn_prefill_fp8.hip): tile sizes, the kernel arguments, the LDS
// swizzle of activation rows, the tile schedule and the grid size.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace moe4 {
namespace prefill {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kTq = 192;  // rows of a three-quarter tile
constexpr int kThreads = 256;
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
  // FP16-activation form of the W4A16 up projection only:
  const int32_t* xexp;      // per token: act holds x * 2^-xexp[t] as FP16
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
      f = wave_incl_sum(f);
      t = wave_incl_sum(t);
      h = wave_incl_sum(h);
      incl_f[c] = carry_f + f;
      incl_t[c] = carry_t + t;
      incl_h[c] = carry_h + h;
      carry_f += __builtin_amdgcn_readlane(f, 63);
      carry_t += __builtin_amdgcn_readlane(t, 63);
      carry_h += __builtin_amdgcn_readlane(h, 63);
    }
    int q, cls;
    place(carry_f * a.n_tiles, carry_t * a.n_tiles, carry_h * a.n_tiles, q, cls);
    if (q >= 0) {
      const int m = q / a.n_tiles;
      nt = q % a.n_tiles;
#pragma unroll
      for (int c = 0; c < kMaxExperts / 64; ++c) {
        const int e = 64 * c + lane;
        int f, t, h;
        classes(count[c], f, t, h);
        const int own = cls == 0 ? f : (cls == 1 ? t : h);
        const int incl = cls == 0 ? incl_f[c] : (cls == 1 ? incl_t[c] : incl_h[c]);
        const int excl = incl - own;
        const uint64_t hit = __ballot(e < a.G && m >= excl && m < incl);
        if (hit && g < 0) {
          const int src = __ffsll((long long)hit) - 1;  // wave-uniform
          g = 64 * c + src;
          const int mt = cls ? 0 : m - __builtin_amdgcn_readlane(excl, src);
          r0 = __builtin_amdgcn_readlane(first[c], src);  // from the counting loads
          const int cnt = __builtin_amdgcn_readlane(count[c], src);
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

// Upper bound on the M-tiles of a launch (the grid is sized from it).
inline long long m_tile_bound(const int32_t* offsets, int T, int k, int G) {
  if (!offsets) return (T + BM - 1) / BM;
  return ((long long)T * k + BM - 1) / BM + G;  // each expert adds at most one partial tile
}

// Grid of a launch: N-tiles per expert, and enough workgroups for every XCD's runs
// (each of its three runs, full, three-quarter and half tiles, may round up by one).
inline dim3 size_grid(GemmArgs& a, bool up, long long m_tiles) {
  a.n_tiles = up ? a.I / 128 : a.N / BN;
  const long long tiles = m_tiles * a.n_tiles;
  a.total = (int)((tiles + kXcds - 1) / kXcds * kXcds) + 3 * kXcds;
  return dim3(a.total);
}

}  // namespace prefill
}  // namespace moe4
