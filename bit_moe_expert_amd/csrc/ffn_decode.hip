// Grouped W4A16 expert FFN for few rows per expert (decode and batched decode).
//
// Decode is bound by reading the touched experts' weights once (the GB10 bandwidth
// budget article, section "Mechanism: decode is bandwidth-bound, prefill is
// compute-bound"); batching raises throughput by sharing each weight read across
// the rows of the batch (same article, "Batching changes the arithmetic"). So the
// kernel streams every touched tile once per 16 rows of its expert and nothing else
// from HBM.
//
// Weights come in the tiled layout (prepack.hip): a 16-row x 128-column tile is 1 KB
// of codes + 128 B of scales, stored in the lane order of the 16x16x32 BF16 MFMA
// operand, so each wave reads a tile with one contiguous 1 KB load and one 128 B load;
// or in the canonical (checkpoint) layout, where the same loads gather 16 rows of 64
// code bytes and 8 scale bytes.
//
// Work split. A wave owns a pair of 16-row blocks (up: a gate block and the matching
// up block, so SwiGLU is applied in registers; down: two consecutive W2 blocks) and
// streams them along K. When the routing leaves too few blocks to fill the chip
// (ksplit > 1), the K range of a pair is split over ksplit waves of the workgroup,
// and their partial sums are added in a fixed order through LDS. Each K step is
// dequantised exactly (code * E4M3 scale has at most 6 significant bits) in registers
// while the next steps' tiles are in flight: into BF16 when the activations come from
// registers, into FP16 when they are staged in LDS (see the staged forms below).
//
// Placement. When the grid is resident at once, the (expert, block pair) units are
// dealt to workgroups with a stride of one round of workgroups (unit = round * C +
// slot, C = min(workgroups, CUs)), so the units of each dispatch slot, and hence of
// each CU, differ by at most one whatever the routing; larger grids give each
// workgroup consecutive units (C = 1). When T*k < E only as many experts as can have
// rows are laid out, and each wave finds its expert among the non-empty ones from the
// offsets.
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
  int compact;              // units index the non-empty experts (T*k < G)
  int slots;                // C: workgroups per round of the placement
  int stage_rows;           // LDS form: activation rows staged (all of act)
  int tiled;                // weights in the tiled layout, else canonical
};

constexpr int kSlices = 4;  // fixed K slices (see the accumulation order below)

// Where a wave's MFMA activation operand comes from.
enum XMode {
  kXRegs = 0,    // global memory, loaded into registers with each K step
  kXAll = 1,     // LDS: all rows of `act`, staged once per workgroup
  kXExpert = 2,  // LDS: the rows of the workgroup's expert, staged per pass
  kXSlice = 3,   // LDS: the rows of the workgroup's expert, staged per pass and K slice
};

// One K step of a wave: its two 16 x 128 weight tiles and, when the activations are
// not staged in LDS, its activation fragment.
template <int kX>
struct Stage {
  u32x4 c0, c1;     // codes of the two blocks (this lane's 16 bytes of each 1 KB tile)
  uint32_t s0, s1;  // two E4M3 scales per block (low half of the loaded dword)
  u32x4 x[4];       // activation row rn, columns 128s + 32kq .. +31
};
template <>
struct Stage<kXAll> {
  u32x4 c0, c1;
  uint32_t s0, s1;
};
template <>
struct Stage<kXExpert> {
  u32x4 c0, c1;
  uint32_t s0, s1;
};
template <>
struct Stage<kXSlice> {
  u32x4 c0, c1;
  uint32_t s0, s1;
};

// The expert of a unit and its rows [r0, r0 + M); M = 0 when there is none.
struct Group {
  int g, r0, M;
};

// Expert slot j -> group. Compact layouts (T*k < G) take the j-th expert (in index
// order) that has rows, found from one round of loads: lane l looks at experts
// 4l .. 4l+3 (G <= 256), a wave scan of the per-lane counts finds the lane holding
// the j-th, and that lane's expert and row range are broadcast.
__device__ __forceinline__ Group find_group(const DecodeArgs& a, int j) {
  if (!a.offsets) return j == 0 ? Group{0, 0, a.T} : Group{0, 0, 0};
  if (!a.compact) {
    if (j >= a.G) return Group{0, 0, 0};
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
  const int incl = wave_incl_sum(cnt);
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
// LDS of the staged form: rows, then one FP32 scale per row (16-byte multiple)
__host__ __device__ constexpr size_t x_stage_bytes(int rows, int K) {
  return (size_t)rows * x_row_stride(K) + (((size_t)rows * 4 + 15) & ~size_t(15));
}

// Wave-wide maximum of non-negative floats (NaN ignored), wave-uniform.
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xf, 0xf, false)));
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The kernel. D = K steps in the register ring: while step s is multiplied, steps
// s+1 .. s+D-1 are in flight. Loads are never skipped (past the end they re-read the
// last step), so the number of loads in flight is the same on every path and the
// compiler's wait counts stay at D-1 stages.
//
// Staged forms (kXAll, kXExpert): the workgroup copies activation rows into LDS and
// the waves read their MFMA operand from there. This frees the 16 registers per stage
// that the fragment otherwise takes, so more weight tiles are in flight. kXAll copies
// all of `act` (the batch's tokens for up, all routed rows for down) once, which lets
// the waves of a workgroup work on different experts; kXExpert copies, per pass, the
// rows of the one expert whose consecutive block pairs the workgroup takes.
// The staged forms also multiply in FP16, which halves the dequantisation work (the
// kernel is close to bound by it): the staged rows are scaled by a power of two each
// (max |x| below 2^15) and converted to FP16, the weights are exact in FP16 (see
// dequant8_f16), and the FP32 outputs are scaled back. Scaling by a power of two
// scales every FP32 partial sum exactly, so the result has the same bits as the BF16
// form as long as a row's values lie within 2^32 of its maximum (smaller ones round
// to FP16 subnormals, a change below 2^-40 of the row's largest term).
// kXSlice stages the expert's rows one fixed K slice at a time (for rows too long to
// stage whole), each (row, slice) with its own power of two; a slice's partial sums are
// scaled back before they are added, which keeps the same bits for the same reason.
template <bool kUp, int D, int kX>
__global__ __launch_bounds__(1024, 1) void ffn_decode_kernel(DecodeArgs a) {
  constexpr bool kLds = kX != kXRegs;
  constexpr bool kSlice = kX == kXSlice;
  constexpr bool kPerExpert = kX == kXExpert || kSlice;  // workgroup = one expert's pairs
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_npass;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar registers)
  const int rn = lane & 15, kq = lane >> 4;
  // 4 waves a workgroup; the all-rows form may run up to 16
  const int nthr = kX == kXAll ? (int)blockDim.x : 256, nw = nthr >> 6;
  const int ksplit = a.ksplit, groups = nw / ksplit;
  const int gi = wave / ksplit, q = wave % ksplit;
  const int K = a.K, NS = K / 128, NB = a.N / 16;
  const int pairs_per_group = kUp ? a.I / 16 : a.N / 32;
  // this wave group's unit: spread over dispatch slots, or the workgroup's `groups`
  // consecutive pairs (of one expert: pairs_per_group is a multiple of 4, and these
  // forms run 4 waves a workgroup)
  const int b = blockIdx.x, C = a.slots;
  const int unit = kPerExpert ? b * groups + gi : ((b / C) * groups + gi) * C + (b % C);
  // All-rows form: the activation rows are in LDS before any weight tile is requested.
  // Their first round (up to 8 chunks of 16 bytes per thread) depends on nothing and
  // goes out before the expert lookup; the lookup waits for it anyway, so the stores
  // that follow wait for nothing. Stores placed after the tiles' loads would wait for
  // the tiles as well (loads return in issue order, and the compiler does not count
  // loads issued under a condition, so it waits for all): that held every workgroup's
  // staging, and with it every wave's first step, until the start-up burst of tiles
  // had arrived (median staging end 6.9 us after entry at T = 8, now 4.7 us).
  constexpr int kU = 8;
  u32x4 pre[kX == kXAll ? kU : 1];
  if constexpr (kX == kXAll) {
    const int cpr = K / 8, total = a.stage_rows * cpr;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = u * nthr + tid;
      const int cc = c < total ? c : 0;
      if (u * nthr < total) pre[u] = reinterpret_cast<const u32x4*>(a.act + (size_t)(cc / cpr) * K)[cc % cpr];
    }
  }
  const Group grp = find_group(a, unit / pairs_per_group);
  if constexpr (kX == kXAll) {
    const int cpr = K / 8, total = a.stage_rows * cpr, xs0 = x_row_stride(K);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = u * nthr + tid;
      if (c < total) *reinterpret_cast<u32x4*>(smem + (size_t)(c / cpr) * xs0 + (c % cpr) * 16) = pre[u];
    }
    // rows beyond the first round (more than 8 chunks a thread), before the tiles too
    for (int c = kU * nthr + tid; c < total; c += nthr)
      *reinterpret_cast<u32x4*>(smem + (size_t)(c / cpr) * xs0 + (c % cpr) * 16) =
          reinterpret_cast<const u32x4*>(a.act + (size_t)(c / cpr) * K)[c % cpr];
    // Nothing is in flight here; an explicit wait tells the compiler so on every path
    // (else a later register write behind a skipped store waits for the tiles).
    __builtin_amdgcn_s_waitcnt(0);
  }
  const int g = grp.g, r0 = grp.r0, M = grp.M;
  const int pair = unit % pairs_per_group;
  // rows per pass: an MFMA's 16, or the staged rows of the expert form
  const int rows_pass = kPerExpert ? a.stage_rows : 16;
  const int npass = (M + rows_pass - 1) / rows_pass;

  // the pair's two blocks (row-block indices within the expert)
  int b0, b1, col0;
  if (kUp) {
    col0 = pair * 16;  // h columns col0..col0+15
    b0 = pair;
    b1 = (a.I + col0) / 16;
  } else {
    col0 = pair * 32;  // y columns col0..col0+31
    b0 = 2 * pair;
    b1 = b0 + 1;
  }
  const size_t tile0 = ((size_t)g * NB + b0) * NS, tile1 = ((size_t)g * NB + b1) * NS;
  // each block's K tiles through a buffer resource covering exactly those tiles, so
  // a step needs one offset register and an access past them would read zeros
  const BufRes rc0 = make_res(a.tcodes + tile0 * 1024, NS * 1024);
  const BufRes rc1 = make_res(a.tcodes + tile1 * 1024, NS * 1024);
  const BufRes rs0 = make_res(a.tscales + tile0 * 128, NS * 128);
  const BufRes rs1 = make_res(a.tscales + tile1 * 128, NS * 128);
  // Both layouts keep a 16-row block's codes (16 * K/2 bytes) and scales (16 * K/16)
  // in one contiguous range at the same place; within it, this lane's 16 code bytes
  // and 2 scale bytes of K step s sit at s * step + lane offset: tiled, one 1 KB +
  // 128 B tile per step in lane order; canonical, row rn's 64 code bytes and 8 scale
  // bytes of the step, columns 32kq..32kq+31 of them.
  const int c_lane = a.tiled ? lane * 16 : rn * (K / 2) + kq * 16;
  const int s_lane = a.tiled ? lane * 2 : rn * (K / 16) + kq * 2;
  const int c_step = a.tiled ? 1024 : 64, s_step = a.tiled ? 128 : 8;
  // K is cut into kSlices fixed slices whose partial sums are always added as
  // ((s0 + s1) + s2) + s3, whichever waves computed them: the bits of a row do not
  // depend on ksplit, i.e. on how many tokens share the call.
  const int nsl = kSlices / ksplit, first = q * nsl;
  const int s_begin = first * NS / kSlices, s_end = (first + nsl) * NS / kSlices;
  const int NSL = NS / kSlices;  // K steps per slice (kXSlice: a multiple of D)
  const int xs = x_row_stride(kSlice ? K / kSlices : K);
  // LDS: staged rows, their FP32 scales, then the slices of waves q > 0 handed to
  // wave 0 ([groups][kSlices - nsl][2][64] float4)
  float4* red = reinterpret_cast<float4*>(smem + (kLds ? x_stage_bytes(a.stage_rows, K) : 0));
  float* row_scale = reinterpret_cast<float*>(smem + (size_t)a.stage_rows * xs);

  Stage<kX> st[D];
  const uint16_t* arow = nullptr;
  // steps past the wave's range re-read its last step; a wave with an empty range
  // (NS < kSlices) reads step 0 and never uses it: every wave issues the same loads,
  // so the wait counts after them do not depend on the path taken
  auto issue = [&](Stage<kX>& t, int s) {
    s = s < s_end ? s : s_end - 1;
    s = s > 0 ? s : 0;
    const int co = s * c_step + c_lane, so = s * s_step + s_lane;
    t.c0 = load_b128_nt(rc0, co);
    t.c1 = load_b128_nt(rc1, co);
    t.s0 = load_b16(rs0, so);
    t.s1 = load_b16(rs1, so);
    if constexpr (!kLds) {
#pragma unroll
      for (int j = 0; j < 4; ++j) t.x[j] = *reinterpret_cast<const u32x4*>(arow + s * 128 + 8 * j);
    }
  };
  // the activation row of pass row rn (rows past the pass's real rows use the pass's
  // first row: MFMA rows are independent and those rows are not stored): the routed
  // pair's index for up (row_src divides it by k) or the routed row for down
  auto row_pair = [&](int pass) {
    const int nr = min(rows_pass, M - pass * rows_pass);
    const int r = r0 + pass * rows_pass + (rn < nr ? rn : 0);
    return kUp && a.perm_src ? a.perm_src[r] : r;
  };
  auto row_src = [&](int pair_or_row) { return kUp && a.perm_src ? pair_or_row / a.k : pair_or_row; };

  // copy columns [k0, k0 + kc) of act rows srcrow(i), i < nrows, into LDS rows i, then
  // convert them in place to FP16, each scaled by 2^-sh so that its max |x| is below
  // 2^15, keeping 2^sh in row_scale (the caller synchronises before and after)
  auto stage_rows = [&](int nrows, auto srcrow, int k0, int kc) {
    const int cpr = kc / 8;  // 16-byte chunks per row
    const int total = nrows * cpr;
    // 8 chunks per thread: all loads, then all stores
    auto store8 = [&](int base, const u32x4* buf) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = base + u * nthr + tid;
        if (c < total) *reinterpret_cast<u32x4*>(smem + (size_t)(c / cpr) * xs + (c % cpr) * 16) = buf[u];
      }
    };
    auto copy8 = [&](int base) {
      u32x4 buf[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = base + u * nthr + tid;
        const int cc = c < total ? c : 0;
        buf[u] = reinterpret_cast<const u32x4*>(a.act + (size_t)srcrow(cc / cpr) * K + k0)[cc % cpr];
      }
      store8(base, buf);
    };
    if constexpr (kSlice) {
      // straight into LDS, every load of the slice in flight at once: a wave moves 1 KB
      // blocks (lane l's 16 bytes land at block + 16 l), a row's slice being kc / 512
      // of them
      const int bpr = kc / 512;
      for (int bi = wave; bi < nrows * bpr; bi += nw) {
        const int r = bi / bpr, h = bi % bpr;
        const uint16_t* src = a.act + (size_t)srcrow(r) * K + k0 + h * 512 + lane * 8;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(smem + (size_t)r * xs + h * 1024),
                                         16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      // the first round outside the loop: a loop head would wait for every load in
      // flight (the weight tiles issued before included) before reusing its registers
      if constexpr (kX != kXAll) {  // the all-rows form copied its rows at the start
        copy8(0);
        for (int base = kU * nthr; base < total; base += kU * nthr) copy8(base);
      }
    }
    __syncthreads();
    for (int row = wave; row < nrows; row += nw) {  // wave w converts rows w, w+nw, ...
      uint8_t* rp = smem + (size_t)row * xs;
      float mx = 0.f;
      for (int c = lane; c < cpr; c += 64) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(rp + c * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(v[e])), fabsf(bf16_hi(v[e]))));
      }
      mx = wave_max_f32(mx);
      int sh = __builtin_amdgcn_frexp_expf(mx) - 15;  // mx < 2^(sh + 15)
      sh = sh < -100 ? -100 : (sh > 100 ? 100 : sh);
      const float down = __builtin_ldexpf(1.0f, -sh);
      for (int c = lane; c < cpr; c += 64) {
        u32x4 v = *reinterpret_cast<const u32x4*>(rp + c * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 h = {(_Float16)(bf16_lo(v[e]) * down), (_Float16)(bf16_hi(v[e]) * down)};
          v[e] = __builtin_bit_cast(uint32_t, h);
        }
        *reinterpret_cast<u32x4*>(rp + c * 16) = v;
      }
      if (lane == 0) row_scale[row] = __builtin_ldexpf(1.0f, sh);
    }
  };

  // Staged forms: pass 0's row index, then its first tiles go out, before the
  // activation copy of the per-expert forms, so the round trips overlap (the index is
  // waited for only where it is used, after the copy's loads have been issued)
  int src = 0, pair0 = 0;
  if (kLds && npass > 0) {
    pair0 = row_pair(0);
#pragma unroll
    for (int i = 0; i < D - 1; ++i) issue(st[i], s_begin + i);
  }
  // passes of the workgroup: the most of its groups (the K-split hand-over and the
  // expert form's copies are workgroup barriers, so every wave runs as many passes)
  if (tid == 0) s_npass = 0;
  __syncthreads();
  if (lane == 0 && q == 0 && npass > 0) atomicMax(&s_npass, npass);
  if constexpr (kX == kXAll) {
    stage_rows(a.stage_rows, [&](int i) { return i; }, 0, K);
    __syncthreads();
  }
  __syncthreads();
  const int npass_wg = s_npass;
  if (npass_wg == 0) return;  // workgroup-uniform
  const float ts = M > 0 ? a.tscale[g] : 0.f;

  for (int pass = 0; pass < npass_wg; ++pass) {
    const bool active = pass < npass;  // wave-group-uniform
    const int nr = active ? min(rows_pass, M - pass * rows_pass) : 0;  // real rows in this pass
    if constexpr (kX == kXExpert) {
      // the expert's rows of this pass (one expert per workgroup: all waves agree)
      if (pass > 0) {
        __syncthreads();  // the previous pass's reads are done
        pair0 = row_pair(pass);
      }
      stage_rows(nr, [&](int i) { return row_src(__shfl(pair0, i)); }, 0, K);
      __syncthreads();
    }
    // the expert's rows of this pass, K slice `slc` (the caller synchronises before)
    auto stage_slice = [&](int slc) {
      stage_rows(nr, [&](int i) { return row_src(__shfl(pair0, i)); }, slc * (K / kSlices), K / kSlices);
      __syncthreads();
    };
    if constexpr (kSlice) {
      if (pass > 0) {
        __syncthreads();  // the previous pass's reads are done
        pair0 = row_pair(pass);
      }
      stage_slice(0);
    }
    f32x4 tot0 = {0.f, 0.f, 0.f, 0.f}, tot1 = tot0;
    if (active) {
      if constexpr (kX == kXAll) {
        if (pass == 0) src = row_src(pair0);
      }
      if (!kLds || pass > 0) {  // the staged forms primed pass 0 before their copy
        src = row_src(row_pair(pass));
        arow = a.act + (size_t)src * K + kq * 32;
#pragma unroll
        for (int i = 0; i < D - 1; ++i) issue(st[i], s_begin + i);
      }
      // LDS row: the staged token/row (all rows) or the pass row (expert rows)
      const int lrow = kPerExpert ? (rn < nr ? rn : 0) : src;
      const uint8_t* xl = smem + (size_t)lrow * xs + kq * 64;
      // acc: the running slice; tot: slices first..current, summed in order (wave q = 0)
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
      auto compute = [&](const Stage<kX>& t, int s) {
        u32x4 xv[4];
        if constexpr (kLds) {
#pragma unroll
          for (int j = 0; j < 4; ++j) xv[j] = *reinterpret_cast<const u32x4*>(xl + (kSlice ? s % NSL : s) * 256 + 16 * j);
          const f16x2 sa = e4m3x2_to_f16(t.s0), sb = e4m3x2_to_f16(t.s1);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc0 = mfma16x16x32_f16(xv[j], dequant8_f16(t.c0[j], j < 2 ? sa[0] : sa[1]), acc0);
            acc1 = mfma16x16x32_f16(xv[j], dequant8_f16(t.c1[j], j < 2 ? sb[0] : sb[1]), acc1);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) xv[j] = t.x[j];
          const float sa0 = e4m3_to_f32<0>(t.s0), sa1 = e4m3_to_f32<1>(t.s0);
          const float sb0 = e4m3_to_f32<0>(t.s1), sb1 = e4m3_to_f32<1>(t.s1);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc0 = mfma16x16x32(xv[j], dequant8(t.c0[j], j < 2 ? sa0 : sa1), acc0);
            acc1 = mfma16x16x32(xv[j], dequant8(t.c1[j], j < 2 ? sb0 : sb1), acc1);
          }
        }
      };
      // close slice `sl`: wave 0 adds it to its running total; other waves hand it over
      auto close_slice = [&](int sl) {
        if constexpr (kSlice) {  // scale the slice back first (exact: powers of two)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sc = row_scale[4 * kq + i < nr ? 4 * kq + i : 0];
            tot0[i] += acc0[i] * sc;
            tot1[i] += acc1[i] * sc;
          }
        } else if (q == 0) {
          tot0 += acc0;
          tot1 += acc1;
        } else {
          float4* r = red + ((size_t)(gi * (kSlices - nsl) + (sl - nsl)) * 2) * 64;
          r[lane] = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
          r[64 + lane] = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
        }
        acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1 = acc0;
      };
      int sl = first;
      if (s_begin < s_end) {
        while (sl < first + nsl && (sl + 1) * NS / kSlices <= s_begin) close_slice(sl++);  // empty slices
        for (int sb = s_begin; sb < s_end; sb += D) {
          if constexpr (kSlice) {
            if (sb > s_begin && sb % NSL == 0) {  // the next slice's rows
              __syncthreads();  // every wave is done with the previous slice
              stage_slice(sb / NSL);
            }
          }
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
    }

    if (ksplit > 1) {
      __syncthreads();
      if (active && q == 0) {
        for (int w = nsl; w < kSlices; ++w) {  // the other waves' slices, in order
          const float4* r = red + ((size_t)(gi * (kSlices - nsl) + (w - nsl)) * 2) * 64;
          const float4 u0 = r[lane], u1 = r[64 + lane];
          tot0[0] += u0.x; tot0[1] += u0.y; tot0[2] += u0.z; tot0[3] += u0.w;
          tot1[0] += u1.x; tot1[1] += u1.y; tot1[2] += u1.z; tot1[3] += u1.w;
        }
      }
      __syncthreads();
    }
    if (active && q == 0) {
      const int mbase = 4 * kq;  // pass rows mbase..mbase+3, column rn
      if constexpr (kLds && !kSlice) {  // undo the rows' FP16 scaling (exact: powers of two)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // lane mbase+i holds pass row mbase+i's staged row (all-rows form)
          const int srow = __shfl(src, mbase + i);
          const float sc = row_scale[kX == kXExpert ? (mbase + i < nr ? mbase + i : 0) : srow];
          tot0[i] *= sc;
          tot1[i] *= sc;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mbase + i < nr) {
          const size_t row = (size_t)(r0 + pass * rows_pass + mbase + i);
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

// all_rows: rows of `act` (T for up, the routed rows for down); expert_rows: the most
// rows one expert can have in a decode batch (T: a token routes to an expert once)
hipError_t launch(bool up, const DecodeArgs& base, long long active_groups, int G, long long all_rows,
                  long long expert_rows, hipStream_t s) {
  DecodeArgs a = base;
  a.G = G;
  // when fewer experts can have rows than exist, units only for as many as can
  a.compact = active_groups < G;
  const long long pairs_per_group = up ? a.I / 16 : a.N / 32;
  const long long pairs = active_groups * pairs_per_group;
  // the activation source: all rows in LDS if they fit, else each expert's rows
  // (at most 16 per pass), else registers
  const int rows_alloc = (int)std::min<long long>(expert_rows, 16);
  // routed rows per expert on average (all_rows counts tokens for routed up, routed rows
  // for down, the group's rows for a dense call)
  const long long routed = up && a.offsets ? all_rows * a.k : all_rows;
  const long long avg_rows = a.offsets ? (routed + G - 1) / G : routed;
  int mode = kXRegs;
  int stage_rows = 0;
  if (x_stage_bytes((int)std::min<long long>(all_rows, 1 << 20), a.K) <= kXLdsMaxBytes) {
    mode = kXAll;
    stage_rows = (int)all_rows;
  } else if (x_stage_bytes(rows_alloc, a.K) <= kXLdsMaxBytes) {
    mode = kXExpert;
    stage_rows = rows_alloc;
  } else if (avg_rows <= 4 && x_stage_bytes(8, a.K) <= kXLdsMaxBytes) {
    // few rows per expert: passes of 8 staged rows beat per-slice staging (measured at
    // the decode shape H = 2048: 2.0-2.7 us per layer faster for 16 to 64 tokens; with
    // 8 rows per expert on average the second passes made it 18 us slower)
    mode = kXExpert;
    stage_rows = 8;
  } else if (a.K % (kSlices * 128 * kStagesLds) == 0 && x_stage_bytes(rows_alloc, a.K / kSlices) <= kXLdsMaxBytes) {
    mode = kXSlice;  // a slice's steps are whole rounds of the ring
    stage_rows = rows_alloc;
  }
  // The down projection of a small batch (at most 64 routed rows, i.e. decode up to
  // T*k = 64) reads its few h rows straight from the cache: staging them costs each
  // workgroup a copy and a conversion (a chain of barriers) before its first MFMA, more
  // than the BF16 form's extra dequantisation (measured: -1.9 us per layer at T = 1,
  // -1.1 us at T = 8; up is faster staged).
  if (!up && all_rows <= 64) {
    mode = kXRegs;
    stage_rows = 0;
  }
  a.stage_rows = stage_rows;
  const size_t x_bytes =
      mode == kXRegs ? 0 : x_stage_bytes(stage_rows, mode == kXSlice ? a.K / kSlices : a.K);
  // K split: the most waves per pair for which the whole grid is resident at once,
  // so that every wave starts in the first wave of dispatch and no second, partial
  // round of waves trails behind (a wave's lifetime is a few memory latencies)
  auto lds_bytes = [&](int ks) {
    const size_t red = ks > 1 ? (size_t)(4 / ks) * (kSlices - kSlices / ks) * 2 * 64 * 16 : 0;
    return x_bytes + red;
  };
  const int cus = cu_count();
  auto resident_waves = [&](int ks) {
    const size_t lds = lds_bytes(ks);
    long long wg_per_cu = kWavesPerSimd;  // 4 waves per workgroup, one per SIMD
    if (lds > 0) wg_per_cu = std::min<long long>(wg_per_cu, (long long)(kLdsPerCu / lds));
    return (long long)cus * wg_per_cu * 4;
  };
  int ks = 1;
  for (int cand : {4, 2}) {
    if (mode == kXSlice) break;  // the workgroup's waves go through the slices together
    if (pairs * cand <= resident_waves(cand)) {
      ks = cand;
      break;
    }
  }
  a.ksplit = ks;
  const bool one_round = pairs * ks <= resident_waves(ks);
  // Waves per workgroup: 4, except for the all-rows form with one wave per pair in a
  // single round, which takes one workgroup per CU of up to 16 waves, so that each CU
  // copies and converts the activation rows once instead of once per 4 waves (measured
  // at T = 8: up 20.9 us against 21.4 us with 4-wave groups).
  // (The K-split hand-over buffer is sized for 4 waves; it is only used when ks > 1.)
  int nw = 4;
  if (mode == kXAll && ks == 1 && one_round)
    nw = (int)std::min<long long>(16, std::max<long long>(4, (pairs + cus - 1) / cus));
  const long long groups_per_wg = nw / ks;
  const long long wgs = (pairs + groups_per_wg - 1) / groups_per_wg;
  // a whole number of rounds of `slots` workgroups, so that unit <-> (workgroup,
  // group) is one to one. The spread placement is for grids that are resident at
  // once; larger ones keep consecutive units (the same expert's pairs, whose rows
  // the workgroup's waves share in cache) together (slots = 1). The expert form
  // always takes consecutive units.
  const long long slots = one_round && mode != kXExpert && mode != kXSlice ? std::min<long long>(wgs, cus) : 1;
  a.slots = (int)slots;
  const long long grid = (wgs + slots - 1) / slots * slots;
  const unsigned lds = (unsigned)lds_bytes(ks);
  const dim3 g3((unsigned)grid), b3((unsigned)(64 * nw));
  if (mode == kXAll) {
    if (up) hipLaunchKernelGGL((ffn_decode_kernel<true, kStagesLds, kXAll>), g3, b3, lds, s, a);
    else hipLaunchKernelGGL((ffn_decode_kernel<false, kStagesLds, kXAll>), g3, b3, lds, s, a);
  } else if (mode == kXExpert) {
    if (up) hipLaunchKernelGGL((ffn_decode_kernel<true, kStagesLds, kXExpert>), g3, b3, lds, s, a);
    else hipLaunchKernelGGL((ffn_decode_kernel<false, kStagesLds, kXExpert>), g3, b3, lds, s, a);
  } else if (mode == kXSlice) {
    if (up) hipLaunchKernelGGL((ffn_decode_kernel<true, kStagesLds, kXSlice>), g3, b3, lds, s, a);
    else hipLaunchKernelGGL((ffn_decode_kernel<false, kStagesLds, kXSlice>), g3, b3, lds, s, a);
  } else {
    if (up) hipLaunchKernelGGL((ffn_decode_kernel<true, kStagesReg, kXRegs>), g3, b3, lds, s, a);
    else hipLaunchKernelGGL((ffn_decode_kernel<false, kStagesReg, kXRegs>), g3, b3, lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_up_decode(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                         int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s) {
  if (T == 0) return hipSuccess;
  DecodeArgs a{x, offsets, perm_src, k, T, w13.packed, w13.scales, w13.tscale, 2 * I, H, I, 1, h, G, 0, 1, 0,
               w13.tiled ? 1 : 0};
  const long long active = offsets ? std::min<long long>((long long)T * k, G) : 1;
  return launch(true, a, active, offsets ? G : 1, T, T, s);
}

hipError_t launch_ffn_down_decode(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H, int I,
                           W4View w2, uint16_t* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  DecodeArgs a{h, offsets, nullptr, 1, T, w2.packed, w2.scales, w2.tscale, H, I, I, 1, y, G, 0, 1, 0,
               w2.tiled ? 1 : 0};
  const long long rows = offsets ? (long long)T * k : T;
  const long long active = offsets ? std::min<long long>((long long)T * k, G) : 1;
  return launch(false, a, active, offsets ? G : 1, rows, T, s);
}

}  // namespace moe4
