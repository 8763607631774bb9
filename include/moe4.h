/*
 * libmoe4 — the quantized (W4A16) mixture-of-experts layer on one MI355X (gfx950).
 *
 * The layer is the one the TensorFold issue "GB10: Nemotron decode is 1.4 % (code) /
 * 3.0 % (prose) slower on 1.0.3 than on 1.0.2" (#627) lays out in its Oct 14 comment
 * on where a decode step's time goes: router -> topk -> plan -> routed experts, a
 * shared expert beside them, then add_moe_norm (the weighted MoE sum added to the
 * residual, then normalised). Weights are NVFP4 read as they are stored and computed
 * against BF16 activations, i.e. W4A16 (bear-blog article on TensorFold 1.0.12 /
 * PR804, section "NVFP4 is neither uniform 4-bit nor all-FP4 compute").
 *
 * Storage formats (all row-major and contiguous):
 *   BF16       uint16_t bit patterns.
 *   weights    4-bit E2M1 codes (1 sign, 2 exponent bits with bias 1, 1 mantissa bit),
 *              two per byte along K: element 2j in the low nibble, 2j+1 in the high one.
 *   scales     one OCP FP8 E4M3FN code (bias 7, max 448, 0x7F/0xFF NaN) per 16
 *              consecutive weights along K.
 *   tscale     one FP32 tensor scale per expert matrix.
 *   weight[n][k] = e2m1(code[n][k]) * e4m3(scale[n][k/16]) * tscale.
 *   W13 (per expert): N = 2I rows, K = H; rows 0..I-1 are the gate, I..2I-1 the up
 *   projection.  W2 (per expert): N = H rows, K = I.  The shared expert uses the same
 *   layouts with one expert.
 *
 * Weight layouts. The layout above is the CANONICAL (checkpoint) layout: NVFP4 as a
 * checkpoint stores it, read as is without re-quantisation (bear-blog article on
 * TensorFold 1.0.12 / PR804, section "What PR804 does and does not do"). The expert
 * FFN entry points accept it, and also the TILED layout that moe4_prepack_w4
 * produces from it once, at weight-load time: the same bytes, moved so that every
 * 16-row x 128-column tile is 1 KB of codes plus 128 B of scales in the order the
 * MFMA operands consume them, which streams faster (one contiguous 1 KB read per
 * wave instead of 16 rows of 64 bytes). Tile (g, b, s) (expert g, rows 16b..16b+15,
 * columns 128s..128s+127) sits at tile index (g * N/16 + b) * K/128 + s; within it,
 * lane l = rn + 16*kq (rn = l % 16, kq = l / 16) owns code bytes 16l..16l+15 =
 * canonical row 16b+rn, columns 128s+32kq..+31, and scale bytes 2l, 2l+1 = that row's
 * scales for column groups 8s+2kq and 8s+2kq+1. The tensor scales are not moved.
 * Each weight descriptor names its layout (moe4_w4.layout); both give the same bits.
 *
 * The expert FFN is SwiGLU: h = silu(gate . x) * (up . x), y = W2 . h.
 * Routing: softmax over the E logits, the k largest selected (ties -> lower expert
 * index, output in descending order), their probabilities renormalised to sum to 1.
 * Combine: o = residual + sum_j w_j * y_j (+ shared expert output); the normalised
 * output is n = o / sqrt(mean(o^2) + eps) * gamma (RMSNorm).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are caller-owned DEVICE memory, 16-byte aligned, unless a
 *     comment says otherwise; `shape` and the moe4_w4 descriptors are HOST structs.
 *   - The library never allocates, frees or synchronises. Work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the null stream) and runs
 *     asynchronously. Calls enqueue no host-device copies, so they can be captured
 *     into a HIP graph.
 *   - A returned status covers the synchronous argument checks and launch errors.
 *     Faults during execution surface at the caller's next synchronisation.
 *     On any error nothing has been enqueued, except for MOE4_ERR_HIP, where earlier
 *     launches of the same call may already be queued.
 *   - Intermediate precisions: router logits FP32; routing weights FP32; h and y
 *     BF16 (round to nearest even); all sums FP32 in a fixed order, so repeated calls
 *     on the same inputs give identical bytes.
 *   - T == 0 is a valid no-op: after the shape check the call returns MOE4_OK without
 *     looking at any tensor pointer.
 *   - Envelope: T >= 0, 1 <= k <= min(E, 16), 1 <= E <= 256, H % 128 == 0,
 *     I % 128 == 0, 128 <= H <= 16384, 128 <= I <= 16384, n_shared in {0, 1},
 *     T*k < 2^31. Outside it: MOE4_ERR_UNSUPPORTED.
 *   - Thread safety: calls are reentrant; the only global state is a thread-local
 *     error string.
 */
#ifndef MOE4_H
#define MOE4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE4_ABI_VERSION 2

typedef enum {
  MOE4_OK = 0,
  MOE4_ERR_INVALID_ARG = 1, /* null or misaligned pointer, negative size, bad descriptor */
  MOE4_ERR_UNSUPPORTED = 2, /* a shape outside the envelope above */
  MOE4_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MOE4_ERR_HIP = 4          /* a HIP runtime error; see moe4_last_error() */
} moe4_status;

/* Layer shape (host struct). */
typedef struct {
  int32_t T;        /* tokens in this call */
  int32_t H;        /* hidden size */
  int32_t E;        /* routed experts */
  int32_t k;        /* experts per token */
  int32_t I;        /* expert FFN intermediate size */
  int32_t n_shared; /* always-on shared experts: 0 or 1 */
  float eps;        /* RMSNorm epsilon (> 0) */
} moe4_shape;

/* Layout of a weight descriptor's codes and scales. There is no default: a
 * descriptor whose layout is neither value (e.g. a zero-initialised one) is rejected
 * with MOE4_ERR_INVALID_ARG, so bytes of one layout cannot be read as the other
 * without the caller having said so. */
typedef enum {
  MOE4_W4_CANONICAL = 1, /* [G][N][K/2] codes, [G][N][K/16] scales, row-major (checkpoint) */
  MOE4_W4_TILED = 2      /* the same bytes re-laid out by moe4_prepack_w4 (faster to stream) */
} moe4_w4_layout;

/* One grouped 4-bit weight tensor over G experts (host struct of device pointers).
 * packed: G*N*K/2 code bytes and scales: G*N*K/16 E4M3 bytes, both in `layout`;
 * tscale [G] FP32. packed is 16-byte aligned, scales and tscale 4-byte aligned. */
typedef struct {
  const uint8_t* packed;
  const uint8_t* scales;
  const float* tscale;
  int32_t layout; /* a moe4_w4_layout value */
} moe4_w4;

/* Version of this header the library was built from (MOE4_ABI_VERSION). */
int moe4_abi_version(void);

/* Text of the last error on the calling thread ("" if none). Never NULL; owned by the
 * library and valid until the next call on the same thread. */
const char* moe4_last_error(void);

/* Canonical -> tiled re-layout of one grouped 4-bit tensor (lossless; sizes unchanged).
 * Not on the per-token path: call once when weights are loaded.
 *   G, N, K   experts, rows and columns (N % 32 == 0, K % 128 == 0, else
 *             MOE4_ERR_UNSUPPORTED; G*N*K == 0 is a no-op).
 *   codes     device [G][N][K/2] canonical codes (16-byte aligned); scales [G][N][K/16].
 *   tcodes    device out, G*N*K/2 bytes (16-byte aligned); tscales out, G*N*K/16 bytes.
 * Output buffers must not overlap the inputs. */
moe4_status moe4_prepack_w4(int32_t G, int32_t N, int32_t K, const uint8_t* codes,
                            const uint8_t* scales, uint8_t* tcodes, uint8_t* tscales, void* stream);

/* Bytes of workspace moe4_permute needs for `shape` (host, pure; 0 on a bad shape). */
size_t moe4_permute_workspace_bytes(const moe4_shape* shape);

/* Bytes of workspace moe4_layer needs for `shape` (host, pure; 0 on a bad shape). */
size_t moe4_layer_workspace_bytes(const moe4_shape* shape);

/* Router and top-k (#627, Oct 14 comment: "router -> topk"; the BobClawblaw comment
 * of the same day on keeping the router's wide block grid).
 *   x         BF16 [T][H] activations, or NULL.
 *   w_router  BF16 [E][H] router weights, or NULL (both NULL or both set).
 *   logits    FP32 [T][E]: written (logits[t][e] = sum_h x[t][h] * w_router[e][h],
 *             FP32 accumulation) when x is set; read as the given logits otherwise.
 *   topk_idx  int32 [T][k] out: selected experts, descending logit, ties -> lower index.
 *   topk_w    FP32 [T][k] out: renormalised softmax weights of the selected experts.
 * NaN logits give unspecified (but in-range) indices. */
moe4_status moe4_route(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                       float* logits, int32_t* topk_idx, float* topk_w, void* stream);

/* The plan (#627, Oct 14 comment: "plan" between topk and the routed experts): a stable
 * counting sort of the T*k (token, slot) pairs by expert. Flat pair f = t*k + j.
 *   topk_idx  int32 [T][k] in, values in [0, E) (others are undefined behaviour).
 *   offsets   int32 [E+1] out: offsets[e] = number of pairs routed to experts < e.
 *   perm_src  int32 [T*k] out: rows offsets[e]..offsets[e+1]-1 hold expert e's flat
 *             pair indices f in ascending order.
 *   inv       int32 [T*k] out: inv[f] = the row of pair f (perm_src[inv[f]] == f).
 *   ws        device workspace of at least moe4_permute_workspace_bytes(shape). */
moe4_status moe4_permute(const moe4_shape* shape, const int32_t* topk_idx, int32_t* offsets,
                         int32_t* perm_src, int32_t* inv, void* ws, size_t ws_bytes,
                         void* stream);

/* Routed experts "up" and "down" (#627, BobClawblaw comment of Oct 14: the expert up
 * and down kernels are 63 % of decode GPU time), as a grouped W4A16 SwiGLU FFN.
 *   x         BF16 [T][H] activations.
 *   offsets, perm_src  the plan from moe4_permute: row r of expert e (offsets[e] <= r <
 *             offsets[e+1]) takes token perm_src[r] / k. Both NULL selects dense mode:
 *             one group of T rows, row r = token r, through expert 0 of w13/w2 (the
 *             shared expert).
 *   w13, w2   weight descriptors over E experts (dense mode: over 1 expert).
 *   h         BF16 [R][I] out (R = T*k, dense mode R = T): silu(gate) * up per row.
 *   y         BF16 [R][H] out: W2 . h per row, in plan order. */
moe4_status moe4_expert_ffn(const moe4_shape* shape, const uint16_t* x, const int32_t* offsets,
                            const int32_t* perm_src, const moe4_w4* w13, const moe4_w4* w2,
                            uint16_t* h, uint16_t* y, void* stream);

/* The two halves of moe4_expert_ffn, for callers that schedule them apart (and for
 * timing the dominant one alone). Arguments as for moe4_expert_ffn:
 *   moe4_expert_up:   h [R][I] = silu(gate . x[token(r)]) * (up . x[token(r)]).
 *   moe4_expert_down: y [R][H] = W2 . h[r]; offsets NULL selects dense mode (R = T). */
moe4_status moe4_expert_up(const moe4_shape* shape, const uint16_t* x, const int32_t* offsets,
                           const int32_t* perm_src, const moe4_w4* w13, uint16_t* h, void* stream);
moe4_status moe4_expert_down(const moe4_shape* shape, const uint16_t* h, const int32_t* offsets,
                             const moe4_w4* w2, uint16_t* y, void* stream);

/* The up projection's matmul form on FP16 activations (prefill is bound by the matrix
 * units: GB10 bandwidth-budget article, section "Mechanism: decode is bandwidth-bound,
 * prefill is compute-bound"; the weights stay NVFP4 against 16-bit activations, i.e.
 * W4A16: PR804 article, section "NVFP4 is neither uniform 4-bit nor all-FP4 compute").
 * Each activation row is scaled by its own power of two into FP16, where 4-bit weights
 * times their E4M3 scale dequantise in half the instructions BF16 needs.
 *
 * moe4_act_f16: the activation rows in that form.
 *   x         BF16 [rows][K] in; K a multiple of 8, at most 16384.
 *   x16       FP16 [rows][K] out: x[t][k] * 2^-xexp[t], rounded to nearest even.
 *   xexp      int32 [rows] out: the smallest integer for which max_k |x[t][k]| (NaN
 *             ignored) times 2^-xexp[t] is below 2^15; 0 for a row of zeros.
 *   x16 holds x exactly wherever |x[t][k]| >= 2^-31 * max_k |x[t][k]|; smaller values
 *   round to FP16 subnormals or zero. x must be finite (an infinite value leaves the
 *   row's exponent unspecified).
 *   rows == 0 does nothing; rows below 2^31; x and x16 16-byte aligned.
 *
 * moe4_expert_up_f16: moe4_expert_up on x16 / xexp from moe4_act_f16 of x (rows = T).
 *   Always the MFMA GEMM form (H a multiple of 256 and I of 128, else
 *   MOE4_ERR_UNSUPPORTED), whatever the rows per expert. Products and FP32 partial sums
 *   are those of the BF16 form scaled by 2^-xexp exactly, and the epilogue scales them
 *   back, so h has moe4_expert_up's bytes whenever x16 holds x exactly (see above).
 *   Other arguments as for moe4_expert_up. */
moe4_status moe4_act_f16(int64_t rows, int32_t K, const uint16_t* x, uint16_t* x16, int32_t* xexp,
                         void* stream);
moe4_status moe4_expert_up_f16(const moe4_shape* shape, const uint16_t* x16, const int32_t* xexp,
                               const int32_t* offsets, const int32_t* perm_src, const moe4_w4* w13,
                               uint16_t* h, void* stream);

/* add_moe_norm (#627, table "Median time per launch" and the Oct 14 comment).
 *   y         BF16 [T*k][H] expert outputs in plan order.
 *   inv       int32 [T*k] from moe4_permute.
 *   topk_w    FP32 [T][k] routing weights.
 *   shared_y  BF16 [T][H] shared-expert output, or NULL.
 *   residual  BF16 [T][H]; gamma BF16 [H].
 *   residual_out BF16 [T][H] out: o = residual + sum_j topk_w[t][j] * y[inv[t*k+j]]
 *             (+ shared_y[t]), summed in FP32 in the order j = 0..k-1; may alias residual.
 *   normed_out BF16 [T][H] out: o / sqrt(mean(o^2) + eps) * gamma from the FP32 o. */
moe4_status moe4_combine_norm(const moe4_shape* shape, const uint16_t* y, const int32_t* inv,
                              const float* topk_w, const uint16_t* shared_y,
                              const uint16_t* residual, const uint16_t* gamma,
                              uint16_t* residual_out, uint16_t* normed_out, void* stream);

/* The whole layer: route -> permute -> routed expert FFN (+ shared expert FFN when
 * shape->n_shared == 1) -> combine_norm, enqueued on `stream`.
 *   x, w_router, logits   as for moe4_route (w_router NULL: logits are given).
 *   w13, w2               routed expert weights; shared13, shared2 the shared expert
 *                         (required iff n_shared == 1, else ignored).
 *   residual, gamma       as for moe4_combine_norm.
 *   topk_idx, topk_w      int32 / FP32 [T][k] out (the routing decision).
 *   residual_out, normed_out  BF16 [T][H] out.
 *   ws                    device workspace of at least moe4_layer_workspace_bytes(shape);
 *                         it holds the plan, h and y between the steps, and, where the
 *                         up projections run on the GEMM (40 or more rows per expert on
 *                         average; T >= 40 for the shared expert), x in moe4_act_f16's
 *                         form, which those up GEMMs read (same h bytes, see
 *                         moe4_expert_up_f16). */
moe4_status moe4_layer(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                       float* logits, const moe4_w4* w13, const moe4_w4* w2,
                       const moe4_w4* shared13, const moe4_w4* shared2,
                       const uint16_t* residual, const uint16_t* gamma, int32_t* topk_idx,
                       float* topk_w, uint16_t* residual_out, uint16_t* normed_out, void* ws,
                       size_t ws_bytes, void* stream);

/* moe4_layer for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same launches,
 * with the plan, h and y (and the FP16 rows) in a scratch array of
 * MOE4_NOALLOC_SCRATCH_BYTES that the library holds in each GPU's memory for the life
 * of the process, instead of a
 * caller workspace. Arguments as for moe4_layer, without ws and ws_bytes.
 *   - Shapes whose layer workspace (moe4_layer_workspace_bytes) exceeds
 *     MOE4_NOALLOC_SCRATCH_BYTES return MOE4_ERR_UNSUPPORTED (64 MiB holds decode and
 *     batched decode up to a few thousand routed rows, e.g. 256 tokens x top-8 at
 *     H = 4096, I = 2048; prefill shapes need moe4_layer).
 *   - The call allocates and frees nothing. Its first call on a device looks the
 *     array up (hipGetSymbolAddress); make that call outside graph capture.
 *   - Every call on a GPU shares that GPU's array, and each call writes every byte of
 *     it that it reads, so nothing has to be cleared between calls; but calls that
 *     overlap on one GPU (other streams, other threads) race on it: order them. */
#define MOE4_NOALLOC_SCRATCH_BYTES (64u << 20)
moe4_status moe4_layer_noalloc(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                               float* logits, const moe4_w4* w13, const moe4_w4* w2,
                               const moe4_w4* shared13, const moe4_w4* shared2,
                               const uint16_t* residual, const uint16_t* gamma, int32_t* topk_idx,
                               float* topk_w, uint16_t* residual_out, uint16_t* normed_out,
                               void* stream);

/* The whole layer with the routed chain on a side stream (#627, jschmied's comment of
 * Oct 14 on where one step's time goes: the router, top-k, plan and routed experts run
 * on a side stream while the main stream runs the shared expert and then waits for
 * them). Arguments as for moe4_layer, plus:
 *   side_stream  a hipStream_t (as void*) for the router, plan and routed experts.
 *   fork_event, join_event  two hipEvent_t (as void*) owned by the caller: fork_event
 *                is recorded on `stream` and waited for by side_stream before the
 *                chain; join_event is recorded on side_stream after it and waited for
 *                by `stream` before the combine, which runs on `stream`.
 * With n_shared == 0, or side_stream NULL or equal to `stream`, this is moe4_layer
 * (the events are not used). Results are bit-identical to moe4_layer. Missing events
 * with a distinct side stream and a shared expert are MOE4_ERR_INVALID_ARG. The events
 * and streams make the call capturable into a HIP graph as a fork and join. */
moe4_status moe4_layer_side(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                            float* logits, const moe4_w4* w13, const moe4_w4* w2,
                            const moe4_w4* shared13, const moe4_w4* shared2,
                            const uint16_t* residual, const uint16_t* gamma, int32_t* topk_idx,
                            float* topk_w, uint16_t* residual_out, uint16_t* normed_out, void* ws,
                            size_t ws_bytes, void* stream, void* side_stream, void* fork_event,
                            void* join_event);

/* The FP8 (W4A8) prefill variant: the expert FFN with FP8 E4M3 matmul inputs, for
 * prompt processing (the Qiita TensorFold 1.1.x article, section "Why it still does not
 * reach 0.6.6", names an FP8 prompt-matmul option; the PR804 article's NVFP4 section
 * tells W4A16 apart from lower-precision activations). The pages fix neither the
 * activation format nor the weight rounding; this library reads them as follows, and
 * every result is defined by this reading:
 *   - activations (x into the up projection, the BF16 h into the down projection) are
 *     quantised in blocks of 32 consecutive values along K: each block gets a power-of-
 *     two scale 2^e, e the smallest integer for which the block's largest magnitude
 *     times 2^-e is at most 448 (the largest E4M3 value, so nothing saturates; e = 0
 *     for an all-zero block; e clamped to [-127, 127]), and each value times 2^-e is
 *     rounded to E4M3, nearest with ties to even;
 *   - each weight, code * E4M3 block scale (exact), is rounded to E4M3 the same way,
 *     saturating at +-448; the FP32 tensor scale multiplies the FP32 sums;
 *   - h and y are BF16 as in the W4A16 path.
 * Shapes: H a multiple of 256, I a multiple of 128 (else MOE4_ERR_UNSUPPORTED). Inputs
 * must be finite.
 *
 * moe4_quant_mxfp8: the activation quantiser alone.
 *   x         BF16 [rows][K] in; K a multiple of 32.
 *   q         uint8 [rows][K] out: the E4M3 codes (OCP E4M3FN bytes).
 *   e         uint8 [rows][K/32] out: each block's scale as an E8M0 byte, e + 127.
 *   rows == 0 does nothing; x and q 16-byte aligned; rows * K / 32 below 2^39 (one launch),
 *   else MOE4_ERR_UNSUPPORTED. */
moe4_status moe4_quant_mxfp8(int64_t rows, int32_t K, const uint16_t* x, uint8_t* q, uint8_t* e,
                             void* stream);

/* Device workspace moe4_expert_ffn_w4a8 and moe4_layer_w4a8 need (0 for an invalid or
 * unsupported shape). */
size_t moe4_w4a8_workspace_bytes(const moe4_shape* shape);

/* moe4_expert_ffn with the FP8 matmul inputs above. Arguments as for moe4_expert_ffn,
 * plus:
 *   h         BF16 [R][I] out, or NULL (h is then kept only in its FP8 form, in ws).
 *   ws        device workspace of at least moe4_w4a8_workspace_bytes(shape), 16-byte
 *             aligned: it holds x and h in their block-scaled FP8 form. */
moe4_status moe4_expert_ffn_w4a8(const moe4_shape* shape, const uint16_t* x, const int32_t* offsets,
                                 const int32_t* perm_src, const moe4_w4* w13, const moe4_w4* w2,
                                 uint16_t* h, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* The two halves of moe4_expert_ffn_w4a8 on activations already in their FP8 form
 * (for callers that schedule them apart, and for timing the dominant one alone).
 * Arguments as for moe4_expert_ffn_w4a8, plus:
 *   x8, xs    moe4_quant_mxfp8 of x: uint8 [T][H] E4M3 codes (16-byte aligned) and
 *             uint8 [T][H/32] E8M0 scale bytes.
 *   h8, hs    out of moe4_expert_up_w4a8 and in of moe4_expert_down_w4a8: h in the
 *             same form, uint8 [R][I] (16-byte aligned) and uint8 [R][I/32] (R = T*k,
 *             dense mode T), the BF16 h quantised exactly as moe4_quant_mxfp8 does.
 *   h         BF16 [R][I] out of the up half, or NULL. */
moe4_status moe4_expert_up_w4a8(const moe4_shape* shape, const uint8_t* x8, const uint8_t* xs,
                                const int32_t* offsets, const int32_t* perm_src, const moe4_w4* w13,
                                uint16_t* h, uint8_t* h8, uint8_t* hs, void* stream);
moe4_status moe4_expert_down_w4a8(const moe4_shape* shape, const uint8_t* h8, const uint8_t* hs,
                                  const int32_t* offsets, const moe4_w4* w2, uint16_t* y, void* stream);

/* moe4_layer with the routed and the shared expert FFN in the FP8 form above (routing,
 * plan, combine and norm unchanged). Arguments as for moe4_layer; ws is at least
 * moe4_w4a8_workspace_bytes(shape). */
moe4_status moe4_layer_w4a8(const moe4_shape* shape, const uint16_t* x, const uint16_t* w_router,
                            float* logits, const moe4_w4* w13, const moe4_w4* w2,
                            const moe4_w4* shared13, const moe4_w4* shared2,
                            const uint16_t* residual, const uint16_t* gamma, int32_t* topk_idx,
                            float* topk_w, uint16_t* residual_out, uint16_t* normed_out, void* ws,
                            size_t ws_bytes, void* stream);

/* Neighbouring glue: the two RMSNorm launches of a decode step beside the MoE layer
 * (#627: add_rmsnorm in the Oct 10 list of the other glue ops, add_rmsnorm and
 * group_rmsnorm in the Oct 14 per-step breakdown). Neither takes a moe4_shape.
 * Constraints: 0 <= T <= 2^24 (T == 0 does nothing); H a multiple of 8 in [8, 16384]; eps > 0;
 * pointers 16-byte aligned; gamma must not alias an output; each output may alias any
 * input (every element is read before it is written), the two outputs must differ.
 *
 * add_rmsnorm: the residual add and RMSNorm in front of attention.
 *   x, residual  BF16 [T][H] in.
 *   gamma        BF16 [H].
 *   residual_out BF16 [T][H] out: o = x + residual (FP32 sum, rounded to BF16).
 *   normed_out   BF16 [T][H] out: o / sqrt(mean(o^2) + eps) * gamma from the FP32 o. */
moe4_status moe4_add_rmsnorm(int32_t T, int32_t H, const uint16_t* x, const uint16_t* residual,
                             const uint16_t* gamma, float eps, uint16_t* residual_out,
                             uint16_t* normed_out, void* stream);

/* group_rmsnorm: RMSNorm over contiguous groups of `group` columns of each row (the
 * pages name the launch only; read here as each group normalised by its own mean
 * square, then one gamma over the row, with no gate).
 *   x          BF16 [T][H] in.
 *   group      columns per group: a multiple of 8 that divides H (group == H is a plain
 *              RMSNorm).
 *   gamma      BF16 [H].
 *   normed_out BF16 [T][H] out: x / sqrt(mean over x's group(x^2) + eps) * gamma. */
moe4_status moe4_group_rmsnorm(int32_t T, int32_t H, int32_t group, const uint16_t* x,
                               const uint16_t* gamma, float eps, uint16_t* normed_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE4_H */
