// The routing plan: a stable counting sort of the flat (token, slot) pairs by expert.
//
// TensorFold's MoE layer runs "plan" between top-k and the routed experts (issue
// #627, Oct 14 comment on where a step's time goes). Here the plan is a counting
// sort whose every output is unique: offsets (exclusive scan of per-expert counts),
// perm_src (each expert's pair indices in ascending order) and its inverse. Nothing
// is ordered by atomics: counts are integer sums (order-free), and a pair's rank
// among equal experts comes from wave ballots plus per-wave counts in a fixed order,
// so the result is bit-identical run to run.
//
// Small inputs (n <= kSingleMax) use one 1024-thread workgroup for everything;
// larger ones use three launches: per-slice histograms, a scan over (expert, slice),
// and a per-slice stable scatter. For small decode batches the layer can also fuse
// the top-k selection into the one-workgroup plan (route_plan_kernel).
#include "device.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace moe4 {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;   // 16
constexpr int kMaxE = 256;
constexpr long long kSingleMax = 16384;    // one workgroup up to this many pairs
constexpr int kSlice = 4096;               // pairs per slice in the multi-block path
constexpr int kRoutePlanMaxPairs = 16384;  // fused top-k + plan: pairs kept in LDS
// ... and at most 16 tokens (one per wave): with more, the one-workgroup plan is slower
// than the top-k and permute launches it replaces (measured per layer at the decode
// shape, k = 8: 6 us faster separate at 48 tokens, 9 us at 64, 11 us at the batched
// T = 64 workload; the same at 16 tokens)
constexpr int kRoutePlanMaxTokens = 16;

// Exclusive scan of v (one value per thread for threads < 256) across the first four
// waves; returns the exclusive prefix, and the total through *total. Must be called
// by all threads of the block.
__device__ int block_exclusive_scan256(int v, int* lds4, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_sum(v);
  if (wave < 4 && lane == 63) lds4[wave] = incl;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave && w < 4; ++w) pre += lds4[w];
  *total = lds4[0] + lds4[1] + lds4[2] + lds4[3];
  __syncthreads();
  return pre + incl - v;
}

// One round of the stable scatter: thread tid takes pair f = base + tid (if f < end).
// run[e] holds the next free row of expert e; wcnt is [kWaves][E] scratch.
__device__ void scatter_round(const int32_t* __restrict__ flat, long long base, long long end,
                              int E, int* run, int* wcnt, int32_t* __restrict__ perm_src,
                              int32_t* __restrict__ inv) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long f = base + tid;
  const int e = f < end ? flat[f] : -1;
  for (int i = tid; i < kWaves * E; i += kThreads) wcnt[i] = 0;
  // lanes of this wave with the same expert (9 bits: 0..255 and -1 differ)
  uint64_t peers = ~0ull;
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    const int bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(peers & below);
  __syncthreads();
  if (e >= 0 && rank == 0) wcnt[wave * E + e] = __popcll(peers);
  __syncthreads();
  if (e >= 0) {
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wcnt[w * E + e];
    const int dest = run[e] + pre + rank;
    perm_src[dest] = (int32_t)f;
    inv[f] = dest;
  }
  __syncthreads();
  for (int x = tid; x < E; x += kThreads) {
    int s = 0;
    for (int w = 0; w < kWaves; ++w) s += wcnt[w * E + x];
    run[x] += s;
  }
  __syncthreads();
}

// The whole plan in one workgroup: histogram, scan, stable scatter. `flat` may point
// to global memory or LDS.
__device__ void plan_single(const int32_t* flat, int n, int E, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ perm_src, int32_t* __restrict__ inv, int* cnt, int* run,
                            int* wcnt, int* lds4) {
  const int tid = threadIdx.x;
  for (int i = tid; i < E; i += kThreads) cnt[i] = 0;
  __syncthreads();
  for (int f = tid; f < n; f += kThreads) atomicAdd(&cnt[flat[f]], 1);
  __syncthreads();
  const int v = tid < E ? cnt[tid] : 0;
  int total;
  const int pre = block_exclusive_scan256(v, lds4, &total);
  if (tid < E) {
    run[tid] = pre;
    offsets[tid] = pre;
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  for (long long base = 0; base < n; base += kThreads)
    scatter_round(flat, base, n, E, run, wcnt, perm_src, inv);
}

// The plan of at most 64 pairs by one wave, without block barriers: lane f holds pair
// f's expert; the counts go through LDS atomics, their exclusive scan gives the
// offsets (each lane sums 4 consecutive experts, then a wave scan), and a pair's row
// is its expert's offset plus its rank among the lower lanes with the same expert
// (the stable order). `flat` is in LDS; `start` is E ints of LDS scratch.
__device__ void plan_wave(const int* flat, int n, int E, int32_t* __restrict__ offsets,
                          int32_t* __restrict__ perm_src, int32_t* __restrict__ inv, int* start) {
  const int lane = threadIdx.x & 63;
  const int e = lane < n ? flat[lane] : -1;
  for (int i = lane; i < E; i += kWave) start[i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (e >= 0) atomicAdd(&start[e], 1);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // experts 4*lane .. 4*lane+3 (E <= 256)
  int c[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = 4 * lane + j;
    c[j] = x < E ? start[x] : 0;
    sum += c[j];
  }
  const int incl = wave_incl_sum(sum);
  int pre = incl - sum;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int x = 4 * lane + j;
    if (x < E) {
      start[x] = pre;
      offsets[x] = pre;
    }
    pre += c[j];
  }
  if (lane == 63) offsets[E] = incl;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // lanes with the same expert (9 bits: 0..255 and -1 differ)
  uint64_t peers = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const int v = (e >> bit) & 1;
    const uint64_t bal = __ballot(v);
    peers &= v ? bal : ~bal;
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  if (e >= 0) {
    const int dest = start[e] + __popcll(peers & below);
    perm_src[dest] = lane;
    inv[lane] = dest;
  }
}

__global__ __launch_bounds__(kThreads) void permute_single_kernel(const int32_t* __restrict__ flat,
                                                                  int n, int E,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ perm_src,
                                                                  int32_t* __restrict__ inv) {
  __shared__ int cnt[kMaxE];
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kWaves * kMaxE];
  __shared__ int lds4[4];
  plan_single(flat, n, E, offsets, perm_src, inv, cnt, run, wcnt, lds4);
}

// Top-k of every token (wave w takes tokens w, w + 16, ...) followed by the plan, in
// one workgroup: one launch instead of two for small batches. The selections are
// kept in LDS for the plan and written out as the routing outputs. Up to 64 pairs
// (decode up to T*k = 64) the plan is one wave's (plan_wave), without the block
// barriers of the histogram, scan and scatter rounds.
__global__ __launch_bounds__(kThreads) void route_plan_kernel(const float* __restrict__ logits, int T,
                                                              int E, int k, int32_t* __restrict__ idx,
                                                              float* __restrict__ w,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm_src,
                                                              int32_t* __restrict__ inv) {
  __shared__ int sidx[kRoutePlanMaxPairs];
  __shared__ int cnt[kMaxE];
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kWaves * kMaxE];
  __shared__ int lds4[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += kWaves) {
    int oi;
    float ow;
    topk_softmax_row(logits + (size_t)t * E, E, k, oi, ow);
    if (lane < k) {
      sidx[t * k + lane] = oi;
      idx[(size_t)t * k + lane] = oi;
      w[(size_t)t * k + lane] = ow;
    }
  }
  __syncthreads();
  if (T * k <= kWave) {
    if (wave == 0) plan_wave(sidx, T * k, E, offsets, perm_src, inv, cnt);
    return;
  }
  plan_single(sidx, T * k, E, offsets, perm_src, inv, cnt, run, wcnt, lds4);
}

// Slice b = pairs [b*kSlice, min(n, (b+1)*kSlice)); hist[b][e] = its count of expert e.
__global__ __launch_bounds__(kThreads) void permute_hist_kernel(const int32_t* __restrict__ flat,
                                                                long long n, int E,
                                                                int* __restrict__ hist) {
  __shared__ int cnt[kMaxE];
  const int tid = threadIdx.x;
  const long long b0 = (long long)blockIdx.x * kSlice;
  const long long b1 = min(n, b0 + kSlice);
  for (int i = tid; i < E; i += kThreads) cnt[i] = 0;
  __syncthreads();
  for (long long f = b0 + tid; f < b1; f += kThreads) atomicAdd(&cnt[flat[f]], 1);
  __syncthreads();
  for (int i = tid; i < E; i += kThreads) hist[(size_t)blockIdx.x * E + i] = cnt[i];
}

// One block: offsets = exclusive scan of per-expert totals; hist[b][e] becomes the
// first row of slice b's pairs of expert e (expert-major, slice-minor order).
__global__ __launch_bounds__(kThreads) void permute_scan_kernel(int* __restrict__ hist, int nb,
                                                                int E,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int lds4[4];
  const int tid = threadIdx.x;
  int tot = 0;
  if (tid < E)
    for (int b = 0; b < nb; ++b) tot += hist[(size_t)b * E + tid];
  int total;
  const int pre = block_exclusive_scan256(tid < E ? tot : 0, lds4, &total);
  if (tid < E) {
    offsets[tid] = pre;
    int run = pre;
    for (int b = 0; b < nb; ++b) {
      const int c = hist[(size_t)b * E + tid];
      hist[(size_t)b * E + tid] = run;
      run += c;
    }
  }
  if (tid == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(const int32_t* __restrict__ flat,
                                                                   long long n, int E,
                                                                   const int* __restrict__ base,
                                                                   int32_t* __restrict__ perm_src,
                                                                   int32_t* __restrict__ inv) {
  __shared__ int run[kMaxE];
  __shared__ int wcnt[kWaves * kMaxE];
  const int tid = threadIdx.x;
  const long long b0 = (long long)blockIdx.x * kSlice;
  const long long b1 = min(n, b0 + kSlice);
  for (int i = tid; i < E; i += kThreads) run[i] = base[(size_t)blockIdx.x * E + i];
  __syncthreads();
  for (long long s = b0; s < b1; s += kThreads) scatter_round(flat, s, b1, E, run, wcnt, perm_src, inv);
}

}  // namespace

size_t permute_workspace_bytes(long long n, int E) {
  if (n <= kSingleMax) return 0;
  const long long nb = (n + kSlice - 1) / kSlice;
  return (size_t)nb * (size_t)E * sizeof(int);
}

bool route_plan_fits(int T, int k) { return T <= kRoutePlanMaxTokens && T * k <= kRoutePlanMaxPairs; }

hipError_t launch_route_plan(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             int32_t* offsets, int32_t* perm_src, int32_t* inv, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(route_plan_kernel, dim3(1), dim3(kThreads), 0, s, logits, T, E, k, idx, w, offsets,
                     perm_src, inv);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, long long n, int E, int32_t* offsets, int32_t* perm_src,
                          int32_t* inv, void* ws, hipStream_t s) {
  if (n <= kSingleMax) {
    hipLaunchKernelGGL(permute_single_kernel, dim3(1), dim3(kThreads), 0, s, idx, (int)n, E, offsets,
                       perm_src, inv);
    return hipGetLastError();
  }
  const int nb = (int)((n + kSlice - 1) / kSlice);
  int* hist = static_cast<int*>(ws);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(kThreads), 0, s, idx, n, E, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kThreads), 0, s, hist, nb, E, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(kThreads), 0, s, idx, n, E, hist, perm_src,
                     inv);
  return hipGetLastError();
}

}  // namespace moe4
