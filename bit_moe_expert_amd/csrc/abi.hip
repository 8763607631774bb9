// libmoe4 C ABI: argument checks, workspace layout and launch order.
// Everything is checked before the first launch, so an invalid call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe4.h"
#include "launch.hpp"

namespace moe4 {
// whether the up projection of a call runs on the MFMA GEMM (defined below)
bool up_uses_gemm(const int32_t* offsets, int T, int k, int G, int H, int I);
}  // namespace moe4

namespace {

thread_local char g_err[512] = "";

moe4_status fail(moe4_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

moe4_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED(p, name)                                                                  \
  do {                                                                                 \
    if ((p) == nullptr) return fail(MOE4_ERR_INVALID_ARG, "%s is NULL", name);         \
    if (!aligned16(p)) return fail(MOE4_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

moe4_status check_shape(const moe4_shape* s) {
  if (s == nullptr) return fail(MOE4_ERR_INVALID_ARG, "shape is NULL");
  if (s->T < 0 || s->H <= 0 || s->E <= 0 || s->k <= 0 || s->I <= 0)
    return fail(MOE4_ERR_INVALID_ARG, "shape has a negative or zero size (T=%d H=%d E=%d k=%d I=%d)",
                s->T, s->H, s->E, s->k, s->I);
  if (!(s->eps > 0.0f)) return fail(MOE4_ERR_INVALID_ARG, "eps must be > 0");
  if (s->n_shared != 0 && s->n_shared != 1)
    return fail(MOE4_ERR_UNSUPPORTED, "n_shared must be 0 or 1 (got %d)", s->n_shared);
  if (s->E > 256) return fail(MOE4_ERR_UNSUPPORTED, "E=%d > 256", s->E);
  if (s->k > 16 || s->k > s->E) return fail(MOE4_ERR_UNSUPPORTED, "k=%d must be <= min(E, 16)", s->k);
  if (s->H % 128 || s->H < 128 || s->H > 16384)
    return fail(MOE4_ERR_UNSUPPORTED, "H=%d must be a multiple of 128 in [128, 16384]", s->H);
  if (s->I % 128 || s->I < 128 || s->I > 16384)
    return fail(MOE4_ERR_UNSUPPORTED, "I=%d must be a multiple of 128 in [128, 16384]", s->I);
  if (s->T > (1 << 20)) return fail(MOE4_ERR_UNSUPPORTED, "T=%d > 2^20", s->T);
  if ((long long)s->T * s->k >= (1LL << 31)) return fail(MOE4_ERR_UNSUPPORTED, "T*k >= 2^31");
  return MOE4_OK;
}

moe4_status check_w4(const moe4_w4* w, const char* name) {
  if (w == nullptr) return fail(MOE4_ERR_INVALID_ARG, "%s descriptor is NULL", name);
  char buf[64];
  snprintf(buf, sizeof(buf), "%s.packed", name);
  NEED(w->packed, buf);
  snprintf(buf, sizeof(buf), "%s.scales", name);
  if (w->scales == nullptr) return fail(MOE4_ERR_INVALID_ARG, "%s is NULL", buf);
  // scale rows are K/16 bytes: 8-byte multiples for K % 128 == 0; the GEMM copies
  // them a dword at a time
  if (reinterpret_cast<uintptr_t>(w->scales) & 3u)
    return fail(MOE4_ERR_INVALID_ARG, "%s is not 4-byte aligned", buf);
  snprintf(buf, sizeof(buf), "%s.tscale", name);
  if (w->tscale == nullptr) return fail(MOE4_ERR_INVALID_ARG, "%s is NULL", buf);
  if (reinterpret_cast<uintptr_t>(w->tscale) & 3u)
    return fail(MOE4_ERR_INVALID_ARG, "%s is not 4-byte aligned", buf);
  if (w->layout != MOE4_W4_CANONICAL && w->layout != MOE4_W4_TILED)
    return fail(MOE4_ERR_INVALID_ARG,
                "%s.layout is %d: must be MOE4_W4_CANONICAL (%d) or MOE4_W4_TILED (%d)", name, w->layout,
                (int)MOE4_W4_CANONICAL, (int)MOE4_W4_TILED);
  return MOE4_OK;
}

moe4::W4View view(const moe4_w4* w) {
  return moe4::W4View{w->packed, w->scales, w->tscale, w->layout == MOE4_W4_TILED};
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct LayerWs {
  size_t offsets, perm_src, inv, perm_ws, h, y, x16, xexp, total;
  bool f16;  // the layer's up GEMMs take FP16 activations (x16, xexp)
};

// The layer's up projections that run on the MFMA GEMM take the activations in FP16
// (moe4_act_f16's form, computed once per call into the workspace).
LayerWs layer_ws_layout(const moe4_shape* s) {
  LayerWs l{};
  const size_t pairs = (size_t)s->T * s->k;
  const size_t rows = pairs + (size_t)s->T * s->n_shared;
  const int32_t plan = 1;  // any non-NULL offsets: the routed call
  l.f16 = moe4::up_uses_gemm(&plan, s->T, s->k, s->E, s->H, s->I) ||
          (s->n_shared && moe4::up_uses_gemm(nullptr, s->T, s->k, 1, s->H, s->I));
  size_t o = 0;
  l.offsets = o; o += align256((size_t)(s->E + 1) * 4);
  l.perm_src = o; o += align256(pairs * 4);
  l.inv = o;      o += align256(pairs * 4);
  l.perm_ws = o;  o += align256(moe4::permute_workspace_bytes((long long)pairs, s->E));
  l.h = o;        o += align256(rows * s->I * 2);
  l.y = o;        o += align256(rows * s->H * 2);
  if (l.f16) {
    l.x16 = o;    o += align256((size_t)s->T * s->H * 2);
    l.xexp = o;   o += align256((size_t)s->T * 4);
  }
  l.total = o;
  return l;
}

// Scratch of moe4_layer_noalloc: one file-scope device array, which every GPU the
// library runs on holds until the process ends. Host code never passes `scratch`
// itself to a kernel or a copy (on the host the name is a stand-in, not a device
// address): the device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch_ptr.
__device__ __align__(256) static uint8_t scratch[MOE4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch` (looked up on the first call on the device).
moe4_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE4_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MOE4_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE4_OK;
}

// Workspace of the FP8 (W4A8) entry points: the plan, the block-scaled FP8 x and h
// (codes and E8M0 scales), and y.
struct W4a8Ws {
  size_t offsets, perm_src, inv, perm_ws, x8, xs, h8, hs, y, total;
};

W4a8Ws w4a8_ws_layout(const moe4_shape* s) {
  W4a8Ws l{};
  const size_t pairs = (size_t)s->T * s->k;
  const size_t rows = pairs + (size_t)s->T * s->n_shared;
  size_t o = 0;
  l.offsets = o;  o += align256((size_t)(s->E + 1) * 4);
  l.perm_src = o; o += align256(pairs * 4);
  l.inv = o;      o += align256(pairs * 4);
  l.perm_ws = o;  o += align256(moe4::permute_workspace_bytes((long long)pairs, s->E));
  l.x8 = o;       o += align256((size_t)s->T * s->H);
  l.xs = o;       o += align256((size_t)s->T * (s->H / 32));
  l.h8 = o;       o += align256(rows * s->I);
  l.hs = o;       o += align256(rows * (s->I / 32));
  l.y = o;        o += align256(rows * s->H * 2);
  l.total = o;
  return l;
}

moe4_status check_w4a8_shape(const moe4_shape* s) {
  if (!moe4::prefill_shape_ok(s->H, s->I))
    return fail(MOE4_ERR_UNSUPPORTED, "the FP8 (W4A8) form needs H %% 256 == 0 and I %% 128 == 0 (H=%d I=%d)",
                s->H, s->I);
  return MOE4_OK;
}

}  // namespace

namespace moe4 {

// Rows per expert (on average) at which the 256-row MFMA tiles of the prefill kernel
// pay off over streaming each weight tile once per 16 rows. Measured per layer: at 48
// rows the GEMM was 25-27% faster at both H = 2048 and H = 4096; at 32 rows it was 7%
// faster at H = 2048 but 6% slower at H = 4096; at 24 rows the streaming kernel won.
constexpr long long kPrefillRowsPerExpert = 40;

static bool use_prefill(const int32_t* offsets, int T, int k, int G, int H, int I) {
  if (!prefill_shape_ok(H, I)) return false;
  const long long rows = offsets ? (long long)T * k : T;
  return rows >= kPrefillRowsPerExpert * (offsets ? G : 1);
}

bool up_uses_gemm(const int32_t* offsets, int T, int k, int G, int H, int I) {
  return use_prefill(offsets, T, k, G, H, I);
}

hipError_t launch_ffn_up(const uint16_t* x, const int32_t* offsets, const int32_t* perm_src, int k,
                         int T, int G, int H, int I, W4View w13, uint16_t* h, hipStream_t s) {
  if (use_prefill(offsets, T, k, G, H, I))
    return launch_ffn_up_prefill(x, offsets, perm_src, k, T, G, H, I, w13, h, s);
  return launch_ffn_up_decode(x, offsets, perm_src, k, T, G, H, I, w13, h, s);
}

hipError_t launch_ffn_down(const uint16_t* h, const int32_t* offsets, int k, int T, int G, int H, int I,
                           W4View w2, uint16_t* y, hipStream_t s) {
  if (use_prefill(offsets, T, k, G, H, I))
    return launch_ffn_down_prefill(h, offsets, k, T, G, H, I, w2, y, s);
  return launch_ffn_down_decode(h, offsets, k, T, G, H, I, w2, y, s);
}

}  // namespace moe4

extern "C" {

int moe4_abi_version(void) { return MOE4_ABI_VERSION; }

const char* moe4_last_error(void) { return g_err; }

moe4_status moe4_prepack_w4(int32_t G, int32_t N, int32_t K, const uint8_t* codes,
                            const uint8_t* scales, uint8_t* tcodes, uint8_t* tscales, void* stream) {
  g_err[0] = 0;
  if (G < 0 || N < 0 || K < 0) return fail(MOE4_ERR_INVALID_ARG, "negative size (G=%d N=%d K=%d)", G, N, K);
  if (N % 32 || K % 128)
    return fail(MOE4_ERR_UNSUPPORTED, "prepack needs N %% 32 == 0 and K %% 128 == 0 (N=%d K=%d)", N, K);
  if ((long long)G * N * K == 0) return MOE4_OK;
  NEED(codes, "codes");
  NEED(tcodes, "tcodes");
  if (scales == nullptr) return fail(MOE4_ERR_INVALID_ARG, "scales is NULL");
  if (tscales == nullptr) return fail(MOE4_ERR_INVALID_ARG, "tscales is NULL");
  hipError_t e = moe4::launch_prepack(codes, scales, G, N, K, tcodes, tscales,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prepack launch");
  return MOE4_OK;
}

size_t moe4_permute_workspace_bytes(const moe4_shape* shape) {
  if (check_shape(shape) != MOE4_OK) return 0;
  return moe4::permute_workspace_bytes((long long)shape->T * shape->k, shape->E);
}

size_t moe4_layer_workspace_bytes(const moe4_shape* shape) {
  if (check_shape(shape) != MOE4_OK) return 0;
  return layer_ws_layout(shape).total;
}

moe4_status moe4_route(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                       float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  if ((x == nullptr) != (w_router == nullptr))
    return fail(MOE4_ERR_INVALID_ARG, "x and w_router must both be set or both be NULL");
  if (x) {
    NEED(x, "x");
    NEED(w_router, "w_router");
  }
  NEED(logits, "logits");
  NEED(topk_idx, "topk_idx");
  NEED(topk_w, "topk_w");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (x) {
    e = moe4::launch_router_logits(x, w_router, logits, shape->T, shape->H, shape->E, s);
    if (e != hipSuccess) return hip_fail(e, "router_logits launch");
  }
  e = moe4::launch_topk_softmax(logits, topk_idx, topk_w, shape->T, shape->E, shape->k, s);
  if (e != hipSuccess) return hip_fail(e, "topk_softmax launch");
  return MOE4_OK;
}

moe4_status moe4_permute(const moe4_shape* shape, const int32_t* topk_idx, int32_t* offsets,
                         int32_t* perm_src, int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  NEED(topk_idx, "topk_idx");
  NEED(offsets, "offsets");
  NEED(perm_src, "perm_src");
  NEED(inv, "inv");
  const long long n = (long long)shape->T * shape->k;
  const size_t need = moe4::permute_workspace_bytes(n, shape->E);
  if (need > 0) {
    if (ws == nullptr || ws_bytes < need)
      return fail(MOE4_ERR_WORKSPACE, "permute needs %zu workspace bytes, got %zu%s", need, ws_bytes,
                  ws ? "" : " (NULL)");
    if (!aligned16(ws)) return fail(MOE4_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  }
  hipError_t e = moe4::launch_permute(topk_idx, n, shape->E, offsets, perm_src, inv, ws,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  return MOE4_OK;
}

moe4_status moe4_expert_ffn(const moe4_shape* shape, const uint16_t* x, const int32_t* offsets,
                            const int32_t* perm_src, const moe4_w4* w13, const moe4_w4* w2,
                            uint16_t* h, uint16_t* y, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  if ((offsets == nullptr) != (perm_src == nullptr))
    return fail(MOE4_ERR_INVALID_ARG, "offsets and perm_src must both be set or both be NULL");
  NEED(x, "x");
  if (offsets) {
    NEED(offsets, "offsets");
    NEED(perm_src, "perm_src");
  }
  if ((st = check_w4(w13, "w13"))) return st;
  if ((st = check_w4(w2, "w2"))) return st;
  NEED(h, "h");
  NEED(y, "y");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool dense = offsets == nullptr;
  const int G = dense ? 1 : shape->E;
  hipError_t e = moe4::launch_ffn_up(x, offsets, perm_src, shape->k, shape->T, G, shape->H, shape->I,
                                     view(w13), h, s);
  if (e != hipSuccess) return hip_fail(e, "ffn up launch");
  e = moe4::launch_ffn_down(h, offsets, shape->k, shape->T, G, shape->H, shape->I, view(w2), y, s);
  if (e != hipSuccess) return hip_fail(e, "ffn down launch");
  return MOE4_OK;
}

moe4_status moe4_expert_up(const moe4_shape* shape, const uint16_t* x, const int32_t* offsets,
                           const int32_t* perm_src, const moe4_w4* w13, uint16_t* h, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  if ((offsets == nullptr) != (perm_src == nullptr))
    return fail(MOE4_ERR_INVALID_ARG, "offsets and perm_src must both be set or both be NULL");
  NEED(x, "x");
  if (offsets) {
    NEED(offsets, "offsets");
    NEED(perm_src, "perm_src");
  }
  if ((st = check_w4(w13, "w13"))) return st;
  NEED(h, "h");
  const int G = offsets ? shape->E : 1;
  hipError_t e = moe4::launch_ffn_up(x, offsets, perm_src, shape->k, shape->T, G, shape->H, shape->I,
                                     view(w13), h, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ffn up launch");
  return MOE4_OK;
}

moe4_status moe4_expert_down(const moe4_shape* shape, const uint16_t* h, const int32_t* offsets,
                             const moe4_w4* w2, uint16_t* y, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  NEED(h, "h");
  if (offsets) NEED(offsets, "offsets");
  if ((st = check_w4(w2, "w2"))) return st;
  NEED(y, "y");
  const int G = offsets ? shape->E : 1;
  hipError_t e = moe4::launch_ffn_down(h, offsets, shape->k, shape->T, G, shape->H, shape->I, view(w2), y,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ffn down launch");
  return MOE4_OK;
}

moe4_status moe4_act_f16(int64_t rows, int32_t K, const uint16_t* x, uint16_t* x16, int32_t* xexp,
                         void* stream) {
  g_err[0] = 0;
  if (rows < 0 || K <= 0) return fail(MOE4_ERR_INVALID_ARG, "negative or zero size (rows=%lld K=%d)", (long long)rows, K);
  if (K % 8 || K > 16384) return fail(MOE4_ERR_UNSUPPORTED, "K=%d must be a multiple of 8, at most 16384", K);
  if (rows >= (1LL << 31)) return fail(MOE4_ERR_UNSUPPORTED, "rows=%lld >= 2^31", (long long)rows);
  if (rows == 0) return MOE4_OK;
  NEED(x, "x");
  NEED(x16, "x16");
  if (xexp == nullptr) return fail(MOE4_ERR_INVALID_ARG, "xexp is NULL");
  if (reinterpret_cast<uintptr_t>(xexp) & 3u) return fail(MOE4_ERR_INVALID_ARG, "xexp is not 4-byte aligned");
  hipError_t e = moe4::launch_act_f16(x, rows, K, x16, xexp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "act_f16 launch");
  return MOE4_OK;
}

moe4_status moe4_expert_up_f16(const moe4_shape* shape, const uint16_t* x16, const int32_t* xexp,
                               const int32_t* offsets, const int32_t* perm_src, const moe4_w4* w13,
                               uint16_t* h, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (!moe4::prefill_shape_ok(shape->H, shape->I))
    return fail(MOE4_ERR_UNSUPPORTED, "the GEMM form needs H %% 256 == 0 and I %% 128 == 0 (H=%d I=%d)", shape->H,
                shape->I);
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  if ((offsets == nullptr) != (perm_src == nullptr))
    return fail(MOE4_ERR_INVALID_ARG, "offsets and perm_src must both be set or both be NULL");
  NEED(x16, "x16");
  if (xexp == nullptr) return fail(MOE4_ERR_INVALID_ARG, "xexp is NULL");
  if (reinterpret_cast<uintptr_t>(xexp) & 3u) return fail(MOE4_ERR_INVALID_ARG, "xexp is not 4-byte aligned");
  if (offsets) {
    NEED(offsets, "offsets");
    NEED(perm_src, "perm_src");
  }
  if ((st = check_w4(w13, "w13"))) return st;
  NEED(h, "h");
  const int G = offsets ? shape->E : 1;
  hipError_t e = moe4::launch_ffn_up_prefill_f16(x16, xexp, offsets, perm_src, shape->k, shape->T, G, shape->H,
                                                 shape->I, view(w13), h, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ffn up (FP16 activations) launch");
  return MOE4_OK;
}

moe4_status moe4_combine_norm(const moe4_shape* shape, const uint16_t* y, const int32_t* inv,
                              const float* topk_w, const uint16_t* shared_y,
                              const uint16_t* residual, const uint16_t* gamma,
                              uint16_t* residual_out, uint16_t* normed_out, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  NEED(y, "y");
  NEED(inv, "inv");
  NEED(topk_w, "topk_w");
  if (shared_y) NEED(shared_y, "shared_y");
  NEED(residual, "residual");
  NEED(gamma, "gamma");
  NEED(residual_out, "residual_out");
  NEED(normed_out, "normed_out");
  hipError_t e = moe4::launch_combine_norm(y, inv, topk_w, shared_y, residual, gamma, residual_out,
                                           normed_out, shape->T, shape->H, shape->k, shape->eps,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine_norm launch");
  return MOE4_OK;
}

static moe4_status rmsnorm_impl(int32_t T, int32_t H, int32_t group, const uint16_t* x,
                                const uint16_t* residual, const uint16_t* gamma, float eps,
                                uint16_t* residual_out, uint16_t* normed_out, void* stream) {
  if (T < 0 || H <= 0 || group <= 0)
    return fail(MOE4_ERR_INVALID_ARG, "negative or zero size (T=%d H=%d group=%d)", T, H, group);
  if (!moe4::rmsnorm_shape_ok(H, group))
    return fail(MOE4_ERR_UNSUPPORTED, "H=%d must be a multiple of 8 in [8, 16384] and group=%d a multiple of 8 dividing it",
                H, group);
  if (T > (1 << 24)) return fail(MOE4_ERR_UNSUPPORTED, "T=%d > 2^24", T);
  if (!(eps > 0.0f)) return fail(MOE4_ERR_INVALID_ARG, "eps must be > 0");
  if (T == 0) return MOE4_OK;  // nothing to read or write
  NEED(x, "x");
  if (residual) NEED(residual, "residual");
  NEED(gamma, "gamma");
  if (residual_out) NEED(residual_out, "residual_out");
  NEED(normed_out, "normed_out");
  if (residual_out == normed_out) return fail(MOE4_ERR_INVALID_ARG, "residual_out and normed_out are the same buffer");
  if (gamma == normed_out || gamma == residual_out) return fail(MOE4_ERR_INVALID_ARG, "gamma aliases an output");
  hipError_t e = moe4::launch_rmsnorm(x, residual, gamma, residual_out, normed_out, T, H, group, eps,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
  return MOE4_OK;
}

moe4_status moe4_add_rmsnorm(int32_t T, int32_t H, const uint16_t* x, const uint16_t* residual,
                             const uint16_t* gamma, float eps, uint16_t* residual_out,
                             uint16_t* normed_out, void* stream) {
  g_err[0] = 0;
  if (T > 0 && residual == nullptr) return fail(MOE4_ERR_INVALID_ARG, "residual is NULL");
  if (T > 0 && residual_out == nullptr) return fail(MOE4_ERR_INVALID_ARG, "residual_out is NULL");
  return rmsnorm_impl(T, H, H, x, residual, gamma, eps, residual_out, normed_out, stream);
}

moe4_status moe4_group_rmsnorm(int32_t T, int32_t H, int32_t group, const uint16_t* x,
                               const uint16_t* gamma, float eps, uint16_t* normed_out, void* stream) {
  g_err[0] = 0;
  return rmsnorm_impl(T, H, group, x, nullptr, gamma, eps, nullptr, normed_out, stream);
}

// The layer on `stream`, or with the routed chain on `side_stream` (see moe4_layer_side).
// With use_scratch the workspace is the library's static scratch (moe4_layer_noalloc);
// it is looked up only after every argument check has passed.
static moe4_status layer_impl(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                              float* logits, const moe4_w4* w13, const moe4_w4* w2,
                              const moe4_w4* shared13, const moe4_w4* shared2, const uint16_t* residual,
                              const uint16_t* gamma, int32_t* topk_idx, float* topk_w,
                              uint16_t* residual_out, uint16_t* normed_out, void* ws, size_t ws_bytes,
                              void* stream, void* side_stream, void* fork_event, void* join_event,
                              bool use_scratch = false) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if (shape->T == 0) return MOE4_OK;  // nothing to read or write
  NEED(x, "x");
  if (w_router) NEED(w_router, "w_router");
  NEED(logits, "logits");
  if ((st = check_w4(w13, "w13"))) return st;
  if ((st = check_w4(w2, "w2"))) return st;
  if (shape->n_shared) {
    if ((st = check_w4(shared13, "shared13"))) return st;
    if ((st = check_w4(shared2, "shared2"))) return st;
  }
  NEED(residual, "residual");
  NEED(gamma, "gamma");
  NEED(topk_idx, "topk_idx");
  NEED(topk_w, "topk_w");
  NEED(residual_out, "residual_out");
  NEED(normed_out, "normed_out");
  const bool two_streams = shape->n_shared && side_stream && side_stream != stream;
  if (two_streams && (!fork_event || !join_event))
    return fail(MOE4_ERR_INVALID_ARG, "a side stream needs fork_event and join_event");
  const LayerWs L = layer_ws_layout(shape);
  if (use_scratch) {
    if (L.total > (size_t)MOE4_NOALLOC_SCRATCH_BYTES)
      return fail(MOE4_ERR_UNSUPPORTED,
                  "moe4_layer_noalloc: this shape needs %zu bytes of scratch, more than the %zu the "
                  "library holds per GPU (use moe4_layer with a workspace)",
                  L.total, (size_t)MOE4_NOALLOC_SCRATCH_BYTES);
    if ((st = scratch_ptr(&ws))) return st;
    ws_bytes = MOE4_NOALLOC_SCRATCH_BYTES;
  }
  if (ws == nullptr || ws_bytes < L.total)
    return fail(MOE4_ERR_WORKSPACE, "layer needs %zu workspace bytes, got %zu%s", L.total, ws_bytes,
                ws ? "" : " (NULL)");
  if (!aligned16(ws)) return fail(MOE4_ERR_INVALID_ARG, "ws is not 16-byte aligned");

  char* base = static_cast<char*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* perm_src = reinterpret_cast<int32_t*>(base + L.perm_src);
  int32_t* inv = reinterpret_cast<int32_t*>(base + L.inv);
  void* perm_ws = base + L.perm_ws;
  uint16_t* h = reinterpret_cast<uint16_t*>(base + L.h);
  uint16_t* y = reinterpret_cast<uint16_t*>(base + L.y);
  const size_t pairs = (size_t)shape->T * shape->k;
  hipStream_t main = static_cast<hipStream_t>(stream);
  // the routed chain runs on the side stream when there is one (the shared expert
  // stays on the main stream, which then waits for the chain before the combine)
  hipStream_t s = two_streams ? static_cast<hipStream_t>(side_stream) : main;
  const int T = shape->T, H = shape->H, E = shape->E, k = shape->k, I = shape->I;
  uint16_t* x16 = L.f16 ? reinterpret_cast<uint16_t*>(base + L.x16) : nullptr;
  int32_t* xexp = L.f16 ? reinterpret_cast<int32_t*>(base + L.xexp) : nullptr;

  hipError_t e;
  if (L.f16) {  // before the fork: both streams' up GEMMs read it
    e = moe4::launch_act_f16(x, T, H, x16, xexp, main);
    if (e != hipSuccess) return hip_fail(e, "act_f16 launch");
  }
  // the up projection: the GEMM on FP16 activations where the GEMM runs
  auto up = [&](const int32_t* offs, const int32_t* psrc, int G, const moe4_w4* w, uint16_t* hh,
                hipStream_t st) {
    if (L.f16 && moe4::up_uses_gemm(offs, T, k, G, H, I))
      return moe4::launch_ffn_up_prefill_f16(x16, xexp, offs, psrc, k, T, G, H, I, view(w), hh, st);
    return moe4::launch_ffn_up(x, offs, psrc, k, T, G, H, I, view(w), hh, st);
  };
  if (two_streams) {
    e = hipEventRecord(static_cast<hipEvent_t>(fork_event), main);
    if (e != hipSuccess) return hip_fail(e, "fork event record");
    e = hipStreamWaitEvent(s, static_cast<hipEvent_t>(fork_event), 0);
    if (e != hipSuccess) return hip_fail(e, "side stream wait");
  }
  if (w_router) {
    e = moe4::launch_router_logits(x, w_router, logits, T, H, E, s);
    if (e != hipSuccess) return hip_fail(e, "router_logits launch");
  }
  if (moe4::route_plan_fits(T, k)) {
    e = moe4::launch_route_plan(logits, T, E, k, topk_idx, topk_w, offsets, perm_src, inv, s);
    if (e != hipSuccess) return hip_fail(e, "route_plan launch");
  } else {
    e = moe4::launch_topk_softmax(logits, topk_idx, topk_w, T, E, k, s);
    if (e != hipSuccess) return hip_fail(e, "topk_softmax launch");
    e = moe4::launch_permute(topk_idx, (long long)pairs, E, offsets, perm_src, inv, perm_ws, s);
    if (e != hipSuccess) return hip_fail(e, "permute launch");
  }
  e = up(offsets, perm_src, E, w13, h, s);
  if (e != hipSuccess) return hip_fail(e, "ffn up launch");
  e = moe4::launch_ffn_down(h, offsets, k, T, E, H, I, view(w2), y, s);
  if (e != hipSuccess) return hip_fail(e, "ffn down launch");
  const uint16_t* shared_y = nullptr;
  if (shape->n_shared) {
    uint16_t* hs = h + pairs * I;
    uint16_t* ys = y + pairs * H;
    e = up(nullptr, nullptr, 1, shared13, hs, main);
    if (e != hipSuccess) return hip_fail(e, "shared ffn up launch");
    e = moe4::launch_ffn_down(hs, nullptr, k, T, 1, H, I, view(shared2), ys, main);
    if (e != hipSuccess) return hip_fail(e, "shared ffn down launch");
    shared_y = ys;
  }
  if (two_streams) {
    e = hipEventRecord(static_cast<hipEvent_t>(join_event), s);
    if (e != hipSuccess) return hip_fail(e, "join event record");
    e = hipStreamWaitEvent(main, static_cast<hipEvent_t>(join_event), 0);
    if (e != hipSuccess) return hip_fail(e, "main stream wait");
  }
  e = moe4::launch_combine_norm(y, inv, topk_w, shared_y, residual, gamma, residual_out, normed_out, T,
                                H, k, shape->eps, main);
  if (e != hipSuccess) return hip_fail(e, "combine_norm launch");
  return MOE4_OK;
}

moe4_status moe4_layer(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                       float* logits, const moe4_w4* w13, const moe4_w4* w2,
                       const moe4_w4* shared13, const moe4_w4* shared2,
                       const uint16_t* residual, const uint16_t* gamma, int32_t* topk_idx,
                       float* topk_w, uint16_t* residual_out, uint16_t* normed_out, void* ws,
                       size_t ws_bytes, void* stream) {
  return layer_impl(shape, x, w_router, logits, w13, w2, shared13, shared2, residual, gamma, topk_idx, topk_w,
                    residual_out, normed_out, ws, ws_bytes, stream, nullptr, nullptr, nullptr);
}

moe4_status moe4_layer_noalloc(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                               float* logits, const moe4_w4* w13, const moe4_w4* w2,
                               const moe4_w4* shared13, const moe4_w4* shared2,
                               const uint16_t* residual, const uint16_t* gamma, int32_t* topk_idx,
                               float* topk_w, uint16_t* residual_out, uint16_t* normed_out,
                               void* stream) {
  return layer_impl(shape, x, w_router, logits, w13, w2, shared13, shared2, residual, gamma, topk_idx, topk_w,
                    residual_out, normed_out, nullptr, 0, stream, nullptr, nullptr, nullptr, true);
}

moe4_status moe4_quant_mxfp8(int64_t rows, int32_t K, const uint16_t* x, uint8_t* q, uint8_t* e, void* stream) {
  g_err[0] = 0;
  if (rows < 0 || K <= 0) return fail(MOE4_ERR_INVALID_ARG, "negative or zero size (rows=%lld K=%d)", (long long)rows, K);
  if (K % 32) return fail(MOE4_ERR_UNSUPPORTED, "K=%d is not a multiple of 32", K);
  if (rows == 0) return MOE4_OK;
  if (rows > (1LL << 31) / (K / 32) * 256)  // one thread per block of 32: the grid stays below 2^31
    return fail(MOE4_ERR_UNSUPPORTED, "rows=%lld x K=%d is too large for one launch", (long long)rows, K);
  NEED(x, "x");
  NEED(q, "q");
  if (e == nullptr) return fail(MOE4_ERR_INVALID_ARG, "e is NULL");
  hipError_t err = moe4::launch_mxfp8_quant(x, rows, K, q, e, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "mxfp8 quant launch");
  return MOE4_OK;
}

size_t moe4_w4a8_workspace_bytes(const moe4_shape* shape) {
  if (check_shape(shape) != MOE4_OK || check_w4a8_shape(shape) != MOE4_OK) return 0;
  return w4a8_ws_layout(shape).total;
}

moe4_status moe4_expert_ffn_w4a8(const moe4_shape* shape, const uint16_t* x, const int32_t* offsets,
                                 const int32_t* perm_src, const moe4_w4* w13, const moe4_w4* w2, uint16_t* h,
                                 uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_w4a8_shape(shape))) return st;
  if (shape->T == 0) return MOE4_OK;
  if ((offsets == nullptr) != (perm_src == nullptr))
    return fail(MOE4_ERR_INVALID_ARG, "offsets and perm_src must both be set or both be NULL");
  NEED(x, "x");
  if (offsets) {
    NEED(offsets, "offsets");
    NEED(perm_src, "perm_src");
  }
  if ((st = check_w4(w13, "w13"))) return st;
  if ((st = check_w4(w2, "w2"))) return st;
  if (h) NEED(h, "h");
  NEED(y, "y");
  const W4a8Ws L = w4a8_ws_layout(shape);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(MOE4_ERR_WORKSPACE, "the FP8 FFN needs %zu workspace bytes, got %zu%s", L.total, ws_bytes,
                ws ? "" : " (NULL)");
  if (!aligned16(ws)) return fail(MOE4_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  char* b = static_cast<char*>(ws);
  uint8_t* x8 = reinterpret_cast<uint8_t*>(b + L.x8);
  uint8_t* xs = reinterpret_cast<uint8_t*>(b + L.xs);
  uint8_t* h8 = reinterpret_cast<uint8_t*>(b + L.h8);
  uint8_t* hs = reinterpret_cast<uint8_t*>(b + L.hs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = shape->T, H = shape->H, I = shape->I, k = shape->k;
  const int G = offsets ? shape->E : 1;
  hipError_t e = moe4::launch_mxfp8_quant(x, T, H, x8, xs, s);
  if (e != hipSuccess) return hip_fail(e, "mxfp8 quant launch");
  e = moe4::launch_ffn_up_prefill_fp8(x8, xs, offsets, perm_src, k, T, G, H, I, view(w13), h, h8, hs, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 ffn up launch");
  e = moe4::launch_ffn_down_prefill_fp8(h8, hs, offsets, k, T, G, H, I, view(w2), y, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 ffn down launch");
  return MOE4_OK;
}

moe4_status moe4_expert_up_w4a8(const moe4_shape* shape, const uint8_t* x8, const uint8_t* xs,
                                const int32_t* offsets, const int32_t* perm_src, const moe4_w4* w13, uint16_t* h,
                                uint8_t* h8, uint8_t* hs, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_w4a8_shape(shape))) return st;
  if (shape->T == 0) return MOE4_OK;
  if ((offsets == nullptr) != (perm_src == nullptr))
    return fail(MOE4_ERR_INVALID_ARG, "offsets and perm_src must both be set or both be NULL");
  NEED(x8, "x8");
  if (xs == nullptr) return fail(MOE4_ERR_INVALID_ARG, "xs is NULL");
  if (offsets) {
    NEED(offsets, "offsets");
    NEED(perm_src, "perm_src");
  }
  if ((st = check_w4(w13, "w13"))) return st;
  if (h) NEED(h, "h");
  NEED(h8, "h8");
  if (hs == nullptr) return fail(MOE4_ERR_INVALID_ARG, "hs is NULL");
  const int G = offsets ? shape->E : 1;
  hipError_t e = moe4::launch_ffn_up_prefill_fp8(x8, xs, offsets, perm_src, shape->k, shape->T, G, shape->H,
                                                 shape->I, view(w13), h, h8, hs, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 ffn up launch");
  return MOE4_OK;
}

moe4_status moe4_expert_down_w4a8(const moe4_shape* shape, const uint8_t* h8, const uint8_t* hs,
                                  const int32_t* offsets, const moe4_w4* w2, uint16_t* y, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_w4a8_shape(shape))) return st;
  if (shape->T == 0) return MOE4_OK;
  NEED(h8, "h8");
  if (hs == nullptr) return fail(MOE4_ERR_INVALID_ARG, "hs is NULL");
  if (offsets) NEED(offsets, "offsets");
  if ((st = check_w4(w2, "w2"))) return st;
  NEED(y, "y");
  const int G = offsets ? shape->E : 1;
  hipError_t e = moe4::launch_ffn_down_prefill_fp8(h8, hs, offsets, shape->k, shape->T, G, shape->H, shape->I,
                                                   view(w2), y, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 ffn down launch");
  return MOE4_OK;
}

moe4_status moe4_layer_w4a8(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router, float* logits,
                            const moe4_w4* w13, const moe4_w4* w2, const moe4_w4* shared13,
                            const moe4_w4* shared2, const uint16_t* residual, const uint16_t* gamma,
                            int32_t* topk_idx, float* topk_w, uint16_t* residual_out, uint16_t* normed_out,
                            void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  moe4_status st = check_shape(shape);
  if (st) return st;
  if ((st = check_w4a8_shape(shape))) return st;
  if (shape->T == 0) return MOE4_OK;
  NEED(x, "x");
  if (w_router) NEED(w_router, "w_router");
  NEED(logits, "logits");
  if ((st = check_w4(w13, "w13"))) return st;
  if ((st = check_w4(w2, "w2"))) return st;
  if (shape->n_shared) {
    if ((st = check_w4(shared13, "shared13"))) return st;
    if ((st = check_w4(shared2, "shared2"))) return st;
  }
  NEED(residual, "residual");
  NEED(gamma, "gamma");
  NEED(topk_idx, "topk_idx");
  NEED(topk_w, "topk_w");
  NEED(residual_out, "residual_out");
  NEED(normed_out, "normed_out");
  const W4a8Ws L = w4a8_ws_layout(shape);
  if (ws == nullptr || ws_bytes < L.total)
    return fail(MOE4_ERR_WORKSPACE, "the FP8 layer needs %zu workspace bytes, got %zu%s", L.total, ws_bytes,
                ws ? "" : " (NULL)");
  if (!aligned16(ws)) return fail(MOE4_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  char* b = static_cast<char*>(ws);
  int32_t* offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* perm_src = reinterpret_cast<int32_t*>(b + L.perm_src);
  int32_t* inv = reinterpret_cast<int32_t*>(b + L.inv);
  uint8_t* x8 = reinterpret_cast<uint8_t*>(b + L.x8);
  uint8_t* xs = reinterpret_cast<uint8_t*>(b + L.xs);
  uint8_t* h8 = reinterpret_cast<uint8_t*>(b + L.h8);
  uint8_t* hs = reinterpret_cast<uint8_t*>(b + L.hs);
  uint16_t* y = reinterpret_cast<uint16_t*>(b + L.y);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = shape->T, H = shape->H, E = shape->E, k = shape->k, I = shape->I;
  const size_t pairs = (size_t)T * k;
  hipError_t e;
  if (w_router) {
    e = moe4::launch_router_logits(x, w_router, logits, T, H, E, s);
    if (e != hipSuccess) return hip_fail(e, "router_logits launch");
  }
  if (moe4::route_plan_fits(T, k)) {
    e = moe4::launch_route_plan(logits, T, E, k, topk_idx, topk_w, offsets, perm_src, inv, s);
    if (e != hipSuccess) return hip_fail(e, "route_plan launch");
  } else {
    e = moe4::launch_topk_softmax(logits, topk_idx, topk_w, T, E, k, s);
    if (e != hipSuccess) return hip_fail(e, "topk_softmax launch");
    e = moe4::launch_permute(topk_idx, (long long)pairs, E, offsets, perm_src, inv, b + L.perm_ws, s);
    if (e != hipSuccess) return hip_fail(e, "permute launch");
  }
  e = moe4::launch_mxfp8_quant(x, T, H, x8, xs, s);
  if (e != hipSuccess) return hip_fail(e, "mxfp8 quant launch");
  e = moe4::launch_ffn_up_prefill_fp8(x8, xs, offsets, perm_src, k, T, E, H, I, view(w13), nullptr, h8, hs, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 ffn up launch");
  e = moe4::launch_ffn_down_prefill_fp8(h8, hs, offsets, k, T, E, H, I, view(w2), y, s);
  if (e != hipSuccess) return hip_fail(e, "fp8 ffn down launch");
  const uint16_t* shared_y = nullptr;
  if (shape->n_shared) {
    uint8_t* h8s = h8 + pairs * I;
    uint8_t* hss = hs + pairs * (I / 32);
    uint16_t* ys = y + pairs * H;
    e = moe4::launch_ffn_up_prefill_fp8(x8, xs, nullptr, nullptr, k, T, 1, H, I, view(shared13), nullptr, h8s,
                                        hss, s);
    if (e != hipSuccess) return hip_fail(e, "shared fp8 ffn up launch");
    e = moe4::launch_ffn_down_prefill_fp8(h8s, hss, nullptr, k, T, 1, H, I, view(shared2), ys, s);
    if (e != hipSuccess) return hip_fail(e, "shared fp8 ffn down launch");
    shared_y = ys;
  }
  e = moe4::launch_combine_norm(y, inv, topk_w, shared_y, residual, gamma, residual_out, normed_out, T, H, k,
                                shape->eps, s);
  if (e != hipSuccess) return hip_fail(e, "combine_norm launch");
  return MOE4_OK;
}

moe4_status moe4_layer_side(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                            float* logits, const moe4_w4* w13, const moe4_w4* w2,
                            const moe4_w4* shared13, const moe4_w4* shared2,
                            const uint16_t* residual, const uint16_t* gamma, int32_t* topk_idx,
                            float* topk_w, uint16_t* residual_out, uint16_t* normed_out, void* ws,
                            size_t ws_bytes, void* stream, void* side_stream, void* fork_event,
                            void* join_event) {
  return layer_impl(shape, x, w_router, logits, w13, w2, shared13, shared2, residual, gamma, topk_idx, topk_w,
                    residual_out, normed_out, ws, ws_bytes, stream, side_stream, fork_event, join_event);
}

}  // extern "C"
