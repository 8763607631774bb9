// Host-side launchers of the libmoe4 kernels (one per kernel family). Each enqueues
// on `stream` and returns the launch status; argument checks happen in abi.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe4 {

// Router GEMV: logits[t][e] = sum_h x[t][h] * wr[e][h] (BF16 in, FP32 accumulate).
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, float* logits, int T, int H,
                                int E, hipStream_t s);

// Top-k selection + renormalised softmax over the selected logits.
hipError_t launch_topk_softmax(const float* logits, int32_t* idx, float* w, int T, int E, int k,
                               hipStream_t s);

// Stable counting sort of flat pair indices by expert.
size_t permute_workspace_bytes(long long n, int E);
hipError_t launch_permute(const int32_t* idx, long long n, int E, int32_t* offsets, int32_t* perm_src,
                          int32_t* inv, void* ws, hipStream_t s);

// Top-k + plan in one workgroup for small batches (route_plan_fits(T, k)).
bool route_plan_fits(int T, int k);
hipError_t launch_route_plan(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                             int32_t* offsets, int32_t* perm_src, int32_t* inv, hipStream_t s);

// Canonical -> tiled weight layout (lossless).
hipError_t launch_prepack(const uint8_t* codes, const uint8_t* scales, int G, int N, int K,
                          uint8_t* tcodes, uint8_t* tscales, hipStream_t s);

// Grouped W4A16 FFN halves; weights in the tiled or the canonical layout.
struct W4View {
  const uint8_t* packed;
  const uint8_t* scales;
  const float* tscale;
  bool tiled;  // tiled (moe4_prepack_w4) layout, else canonical [G][N][K/2] / [G][N][K/16]
};
// h[r] = silu(gate . x[tok(r)]) * (up . x[tok(r)]); offsets/perm_src NULL = dense (G=1, R=T).
// y[r] = W2 . h[r]. The dispatchers pick the decode (streaming) or the prefill (GEMM)
// kernel from the average rows per expert.
hipError_t launch_ffn_up(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                         int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s);
hipError_t launch_ffn_down(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H, int I,
                           W4View w2, uint16_t* y, hipStream_t s);
// few rows per expert: stream each touched weight tile once per 16 rows
hipError_t launch_ffn_up_decode(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                                int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s);
hipError_t launch_ffn_down_decode(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H,
                                  int I, W4View w2, uint16_t* y, hipStream_t s);
// many rows per expert: 256 x 256 MFMA tiles (needs H % 256 == 0, I % 128 == 0)
bool prefill_shape_ok(int H, int I);
hipError_t launch_ffn_up_prefill(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                                 int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s);
hipError_t launch_ffn_down_prefill(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H,
                                   int I, W4View w2, uint16_t* y, hipStream_t s);
// FP16-activation form of the up GEMM: x16 [T][H] = x * 2^-xexp[t] in FP16 (from
// launch_act_f16); the same h as launch_ffn_up_prefill while x16 holds x exactly.
hipError_t launch_ffn_up_prefill_f16(const uint16_t* x16, const int32_t* xexp, const int32_t* offsets,
                                     const int32_t* perm_src, int k, int T, int G, int H, int I, W4View w13,
                                     uint16_t* h, hipStream_t s);
// x [rows][K] BF16 -> x16 [rows][K] FP16 and xexp [rows] (K % 8 == 0, K <= 16384)
hipError_t launch_act_f16(const uint16_t* x, long long rows, int K, uint16_t* x16, int32_t* xexp, hipStream_t s);

// FP8 (W4A8) prefill form: activations as block-scaled E4M3 (32 values per E8M0
// scale), weights rounded to E4M3, block-scaled FP8 MFMAs. x [rows][K] BF16 ->
// q [rows][K] E4M3 + e [rows][K/32] E8M0 (K % 32 == 0).
hipError_t launch_mxfp8_quant(const uint16_t* x, long long rows, int K, uint8_t* q, uint8_t* e, hipStream_t s);
// up: h8/hs (the down projection's FP8 input) always, BF16 h too when h != NULL
hipError_t launch_ffn_up_prefill_fp8(const uint8_t* x8, const uint8_t* xs, const int32_t* offsets,
                                     const int32_t* perm_src, int k, int T, int G, int H, int I, W4View w13,
                                     uint16_t* h, uint8_t* h8, uint8_t* hs, hipStream_t s);
hipError_t launch_ffn_down_prefill_fp8(const uint8_t* h8, const uint8_t* hs, const int32_t* offsets, int k, int T,
                                       int G, int H, int I, W4View w2, uint16_t* y, hipStream_t s);

// o = residual + sum_j w_j * y[inv[t*k+j]] (+ shared); n = rmsnorm(o) * gamma.
hipError_t launch_combine_norm(const uint16_t* y, const int32_t* inv, const float* w,
                               const uint16_t* shared_y, const uint16_t* residual,
                               const uint16_t* gamma, uint16_t* res_out, uint16_t* norm_out, int T,
                               int H, int k, float eps, hipStream_t s);

// o = x (+ residual); n = o / rms(o over each group of `group` columns) * gamma.
// res_out may be NULL. Needs rmsnorm_shape_ok(H, group).
bool rmsnorm_shape_ok(int H, int group);
hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma,
                          uint16_t* res_out, uint16_t* norm_out, int T, int H, int group, float eps,
                          hipStream_t s);

}  // namespace moe4
