"""fp64 CPU oracle of the quantized (W4A16) mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code, table or constant with the HIP
library (``bit_moe_expert_amd``) and imports nothing from it; it takes plain numpy
arrays in the storage formats described below.

What it computes, in the pages' order. The layer is the one the TensorFold issue
"GB10: Nemotron decode is 1.4 % (code) / 3.0 % (prose) slower on 1.0.3 ..." (#627)
describes in its Oct 14 comment on where the time per step goes: router -> topk ->
plan -> routed experts, a shared expert beside them, then the weighted MoE add with
the residual and a norm (``add_moe_norm``, table "Per-launch kernel times").
The weights are NVFP4 read as W4A16: 4-bit float weights with scales, computed
against BF16 activations (bear-blog article on TensorFold 1.0.12 / PR804, section
"NVFP4 is neither uniform 4-bit nor all-FP4 compute"). The issue's maintainers gate
their kernels on the error against a 64-bit reference (#627, description and the
Oct 10 reply); this oracle is such a reference.

Readings where the pages are silent (each is stated again where it is used):
  R1  E2M1 = 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; OCP MX v1.0.
  R2  the block scale is OCP FP8 E4M3FN (bias 7, no infinities, 0x7F/0xFF NaN).
  R3  weight = e2m1(code) * e4m3(block scale) * fp32 tensor scale.
  R4  16-weight blocks run along K (the reduction axis); element 2j is the low nibble.
  R5  W13 rows 0..I-1 are the gate, rows I..2I-1 the up projection; SwiGLU
      h = silu(gate) * up (Shazeer, "GLU Variants Improve Transformer", 2020).
  R6  routing weights = softmax over all experts, top-k selected, renormalised.
  R7  top-k order: larger logit first; equal logits -> lower expert index first.
  R8  the plan (permutation) is the stable counting sort of the flat pair index
      f = t*k + j by expert.
  R9  the shared expert is ungated (weight 1) and sees every token.
  R10 RMSNorm n = o / sqrt(mean(o^2) + eps) * gamma (Zhang & Sennrich, 2019), with
      o = residual + sum_j w_j * y_j (+ shared); both o and n are layer outputs.
  R11 "W4A16 with BF16 activations": the FFN's activations are BF16 values, so the
      hidden h (the down projection's input) and the expert output y are rounded to
      BF16 (nearest, ties to even); every sum and the combine/norm are fp64, and the
      layer outputs o and n are left unrounded.
  R16 add_rmsnorm (#627, the Oct 10 list of the other glue ops and the Oct 14
      per-step breakdown name it without defining it) is the residual add in front
      of attention followed by the RMSNorm of R10: o = x + residual, n = o / rms(o) *
      gamma; both o and n are outputs.
  R17 group_rmsnorm (named the same way) normalises each contiguous group of G
      columns of a row by that group's own mean square, then multiplies by one gamma
      over the whole row; there is no gate (the pages name none). G = H is R10.
  R18 the FP8 prefill variant (W4A8; the Qiita TensorFold 1.1.x article, section
      "Why it still does not reach 0.6.6", names an FP8 prompt-matmul option, and the
      PR804 article's NVFP4 section tells W4A16 from lower-precision activations):
      the FFN's matmul inputs are FP8 E4M3. Activations (x for the up projection, the
      BF16 h for the down projection) are quantised in blocks of 32 consecutive
      values along K, each block with its own power-of-two scale 2^e, e the smallest
      integer for which the block's largest magnitude times 2^-e is at most 448 (no
      saturation; e = 0 for an all-zero block; e clamped to [-127, 127]), the scaled
      values rounded to E4M3 (nearest, ties to even). Weights: each code * block
      scale (exact) rounded to E4M3 the same way, saturating at 448; the tensor scale
      multiplies the sum. Sums are fp64; h and y are BF16 as in R11.

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
(closed forms, library routines, brute force on tiny inputs, invariants); ``layer``
with a shared expert, and ``layer_w4a8``, are pinned against independent torch
compositions, and ``tests/test_oracle_mutations.py`` checks that planted mistakes fail
a pin. ``oracle/w4a4_study.py`` (reading R19, a study of a form the HIP library does not
compute) is pinned by brute force in ``tests/test_w4a4_study.py``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_value", "bf16_round", "e2m1_value", "e4m3_value", "unpack_codes", "dequant",
    "router_logits", "route", "permute", "swiglu_hidden", "swiglu_ffn", "expert_outputs",
    "combine_norm", "add_rmsnorm", "group_rmsnorm", "layer",
    "e4m3_round", "mxfp8_quantize", "dequant_e4m3", "swiglu_hidden_w4a8", "swiglu_ffn_w4a8",
    "layer_w4a8",
]


# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------
def bf16_value(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> fp64. BF16 is the top half of an IEEE binary32."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """fp64 -> the nearest BF16 value (ties to even), returned as fp64.

    BF16 keeps 8 significant bits: with v = m * 2^e (0.5 <= |m| < 1), v * 2^(8-e) is
    rounded to an integer (np.rint rounds half to even). Below the normal range the
    grid stays 2^-133 (the BF16 subnormal step). Finite inputs only.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    e = np.maximum(e, -125)
    return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """4-bit E2M1 code -> fp64 (reading R1).

    Bits s e1 e0 m: exponent field 0 is subnormal (0.5*m), otherwise
    2^(e-1) * (1 + m/2); the sign bit negates (code 8 is -0).
    """
    c = np.asarray(code).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, (e - 1).astype(np.int64)))
    return np.where(s == 1, -mag, mag)


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """8-bit OCP E4M3FN code -> fp64 (reading R2).

    Bits s e3..e0 m2..m0, bias 7: exponent field 0 is subnormal 2^-6 * m/8,
    otherwise 2^(e-7) * (1 + m/8); e=15, m=7 is NaN; there is no infinity.
    """
    c = np.asarray(code).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes; element 2j is the low nibble (R4)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant(packed: np.ndarray, scales: np.ndarray, tscale: float) -> np.ndarray:
    """One expert's 4-bit matrix -> fp64 [N, K] (reading R3).

    ``packed`` is [N, K/2], ``scales`` [N, K/16] E4M3 codes, ``tscale`` the FP32
    tensor scale; weight[n, k] = e2m1(code[n, k]) * e4m3(scales[n, k // 16]) * tscale.
    """
    # decode through the 16 / 256 possible codes (same functions, applied once each)
    codes = unpack_codes(packed)
    block = np.repeat(e4m3_value(np.arange(256))[scales], 16, axis=-1)
    return e2m1_value(np.arange(16))[codes] * block * float(tscale)


# ----------------------------------------------------------------------------
# Router, top-k and the plan (issue #627, Oct 14 comment: router -> topk -> plan)
# ----------------------------------------------------------------------------
def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wr[e, h], BF16 operands, fp64 sums."""
    return bf16_value(x_bits) @ bf16_value(wr_bits).T


def route(logits: np.ndarray, k: int):
    """Top-k experts per token and their weights (readings R6, R7).

    Softmax over all E logits, then the k largest (ties -> lower index), then the
    selected probabilities renormalised to sum to 1. Returns (idx int32 [T,k],
    w fp64 [T,k]) with idx in selection order.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        # sort key: larger logit first, then lower expert index
        order = sorted(range(E), key=lambda e: (-L[t, e], e))[:k]
        idx[t] = order
        sel = p[t, order]
        w[t] = sel / sel.sum()
    return idx, w


def permute(idx: np.ndarray, E: int):
    """The routing plan (reading R8).

    Flat pair f = t*k + j goes to expert idx[t, j]. offsets[e] = number of pairs of
    experts < e; perm_src lists, expert by expert, the flat indices f of that
    expert in ascending order; inv[f] is the position of f in perm_src.
    """
    flat = np.asarray(idx).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    perm_src = np.concatenate(
        [np.flatnonzero(flat == e) for e in range(E)] + [np.zeros(0, dtype=np.int64)]
    ).astype(np.int32)
    inv = np.empty(flat.size, dtype=np.int32)
    inv[perm_src] = np.arange(flat.size, dtype=np.int32)
    return offsets, perm_src, inv


# ----------------------------------------------------------------------------
# Expert FFN (W4A16 SwiGLU), reading R5
# ----------------------------------------------------------------------------
def swiglu_hidden(x: np.ndarray, w13: np.ndarray) -> np.ndarray:
    """a = silu(Wg x) * (Wu x) for each row of x (fp64), silu(g) = g / (1 + e^-g).

    x [R, H]; w13 [2I, H] (gate rows first, then up rows).
    """
    I = w13.shape[0] // 2
    g = x @ w13[:I].T
    u = x @ w13[I:].T
    # e^-g overflows to inf for g < -709; g / inf is then the correct (signed) zero
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def swiglu_ffn(x: np.ndarray, w13: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """y = W2 (silu(Wg x) * (Wu x)) for each row of x; w2 [H, I].

    The BF16 activations of reading R11: h is rounded to BF16 before the down
    projection and y is rounded to BF16; the sums are fp64.
    """
    h = bf16_round(swiglu_hidden(x, w13))
    return bf16_round(h @ w2.T)


def expert_outputs(x_bits, idx, w13, w2, tokens=None, cache=None) -> np.ndarray:
    """y[t, j] = FFN_{idx[t, j]}(x[t]) for the selected tokens (fp64 [len(tokens), k, H]).

    ``w13``/``w2`` are objects with ``packed``, ``scales`` and ``tscale`` arrays
    over experts. Experts are dequantised one at a time; ``cache`` (a dict) may keep
    them between calls.
    """
    idx = np.asarray(idx)
    tokens = np.arange(idx.shape[0]) if tokens is None else np.asarray(tokens)
    x = bf16_value(np.asarray(x_bits)[tokens])
    sel = idx[tokens]
    k = sel.shape[1]
    H = x.shape[1]
    y = np.zeros((len(tokens), k, H), dtype=np.float64)
    for e in np.unique(sel):
        rr, jj = np.nonzero(sel == e)
        W13, W2 = _expert(w13, w2, int(e), cache)
        y[rr, jj] = swiglu_ffn(x[rr], W13, W2)
    return y


def _expert(w13, w2, e, cache):
    if cache is not None and e in cache:
        return cache[e]
    W13 = dequant(w13.packed[e], w13.scales[e], w13.tscale[e])
    W2 = dequant(w2.packed[e], w2.scales[e], w2.tscale[e])
    if cache is not None:
        cache[e] = (W13, W2)
    return W13, W2


# ----------------------------------------------------------------------------
# Weighted combine, residual add and RMSNorm (add_moe_norm), readings R9, R10
# ----------------------------------------------------------------------------
def combine_norm(y, w, residual_bits, gamma_bits, eps, shared=None):
    """o = residual + sum_j w[t,j] * y[t,j] (+ shared[t]); n = o / rms(o) * gamma.

    y fp64 [T, k, H], w [T, k]; returns (o, n) in fp64.
    """
    o = bf16_value(residual_bits) + np.einsum("tj,tjh->th", np.asarray(w, np.float64), y)
    if shared is not None:
        o = o + shared
    ms = np.mean(o * o, axis=1, keepdims=True)
    n = o / np.sqrt(ms + eps) * bf16_value(gamma_bits)[None, :]
    return o, n


# ----------------------------------------------------------------------------
# The neighbouring RMSNorm glue (add_rmsnorm, group_rmsnorm), readings R16, R17
# ----------------------------------------------------------------------------
def group_rmsnorm(x_bits, group, gamma_bits, eps):
    """n[t, h] = x[t, h] / sqrt(mean of x[t, .]^2 over h's group + eps) * gamma[h].

    x_bits BF16 [T, H] (or fp64 values: anything that is not uint16 is taken as
    values), group divides H; returns fp64 [T, H].
    """
    x = np.asarray(x_bits)
    x = bf16_value(x) if x.dtype == np.uint16 else x.astype(np.float64)
    T, H = x.shape
    if group <= 0 or H % group:
        raise ValueError(f"group {group} does not divide H={H}")
    n = np.empty_like(x)
    for g0 in range(0, H, group):
        seg = x[:, g0:g0 + group]
        ms = np.mean(seg * seg, axis=1, keepdims=True)
        n[:, g0:g0 + group] = seg / np.sqrt(ms + eps)
    return n * bf16_value(gamma_bits)[None, :]


def add_rmsnorm(x_bits, residual_bits, gamma_bits, eps):
    """o = x + residual; n = o / sqrt(mean(o^2) + eps) * gamma (fp64 [T, H] each)."""
    o = bf16_value(x_bits) + bf16_value(residual_bits)
    return o, group_rmsnorm(o, o.shape[1], gamma_bits, eps)


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------
def layer(inp, tokens=None, cache=None, logits=None):
    """The whole layer for one call's inputs (an object with the fields of
    ``LayerInputs``: x, residual, gamma, w13, w2, logits or w_router, shared13,
    shared2, w.k, w.E, w.eps).

    With ``tokens`` only those rows are computed (routing, FFN, combine and norm are
    per token, so a subset is exact); the plan is then left out. ``logits``
    overrides the router (for reusing the fp64 logits of a previous call).
    Returns a dict of fp64 / int32 arrays (``y`` the routed experts' outputs [T, k, H],
    ``shared`` the shared expert's output [T, H] or None).
    """
    wl = inp.w
    T = inp.x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    if logits is None:
        if inp.logits is not None:
            logits = np.asarray(inp.logits, dtype=np.float64)[tok]
        else:
            logits = router_logits(np.asarray(inp.x)[tok], inp.w_router)
    idx, w = route(logits, wl.k)
    full_idx = np.zeros((T, wl.k), dtype=np.int32)
    full_idx[tok] = idx
    y = expert_outputs(inp.x, full_idx, inp.w13, inp.w2, tokens=tok, cache=cache)
    shared = None
    if getattr(inp, "shared13", None) is not None:
        W13 = dequant(inp.shared13.packed[0], inp.shared13.scales[0], inp.shared13.tscale[0])
        W2 = dequant(inp.shared2.packed[0], inp.shared2.scales[0], inp.shared2.tscale[0])
        shared = swiglu_ffn(bf16_value(np.asarray(inp.x)[tok]), W13, W2)
    o, n = combine_norm(y, w, np.asarray(inp.residual)[tok], inp.gamma, wl.eps, shared)
    out = {"logits": logits, "idx": idx, "w": w, "y": y, "o": o, "n": n, "tokens": tok,
           "shared": shared}
    if tokens is None:
        out["offsets"], out["perm_src"], out["inv"] = permute(idx, wl.E)
    return out


# ----------------------------------------------------------------------------
# FP8 (W4A8) prefill variant, reading R18
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """fp64 -> the nearest OCP E4M3FN value (ties to even), saturating at +-448.

    E4M3 keeps 4 significant bits for magnitudes from 2^-6 up and a fixed step of
    2^-9 below (subnormals): with |v| = m * 2^e (1 <= m < 2, e >= -6 after
    clamping), |v| * 2^(3-e) is rounded to an integer (np.rint: half to even).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                 # a = f * 2^e with 0.5 <= f < 1
    e = np.maximum(e - 1, -6)          # exponent of the leading bit, subnormals below 2^-6
    r = np.ldexp(np.rint(np.ldexp(a, 3 - e)), e - 3)
    return np.copysign(np.minimum(r, E4M3_MAX), v)


def mxfp8_quantize(x: np.ndarray, block: int = 32):
    """Block-scaled FP8 activations (reading R18): x [..., K] (K a multiple of block)
    -> (q, e): q fp64 [..., K] E4M3 values and e int [..., K/block], x ~ q * 2^e.

    Each block's scale exponent is the smallest e with max|x| * 2^-e <= 448: with
    max|x| = m * 2^E (1 <= m < 2), e = E - 8 when m <= 1.75 (m * 2^8 <= 448) and
    E - 7 otherwise; 0 for an all-zero block; clamped to [-127, 127].
    """
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % block:
        raise ValueError(f"K={K} is not a multiple of {block}")
    xb = x.reshape(x.shape[:-1] + (K // block, block))
    amax = np.max(np.abs(xb), axis=-1)
    f, E = np.frexp(amax)              # amax = (2f) * 2^(E-1), 1 <= 2f < 2
    e = np.where(2.0 * f <= 1.75, E - 1 - 8, E - 1 - 7)
    e = np.where(amax == 0, 0, e)
    e = np.clip(e, -127, 127).astype(np.int64)
    q = e4m3_round(np.ldexp(xb, -e[..., None]))
    return q.reshape(x.shape), e


def _mx_value(x: np.ndarray, block: int = 32) -> np.ndarray:
    q, e = mxfp8_quantize(x, block)
    return (q.reshape(e.shape + (block,)) * np.exp2(e)[..., None]).reshape(q.shape)


def dequant_e4m3(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """One expert's 4-bit matrix with each weight (code * E4M3 block scale, exact)
    rounded to E4M3 (reading R18) -> fp64 [N, K]; the tensor scale is left out (it
    multiplies the sums)."""
    # the rounded product of every (code, scale) pair, taken once each (16 x 256)
    table = e4m3_round(e2m1_value(np.arange(16))[:, None] * e4m3_value(np.arange(256))[None, :])
    codes = unpack_codes(packed)
    sc = np.repeat(np.asarray(scales, dtype=np.uint8), 16, axis=-1)
    return table[codes, sc]


def swiglu_hidden_w4a8(x: np.ndarray, w13_8: np.ndarray, tscale: float) -> np.ndarray:
    """a = silu(g) * u with g, u = tscale * (MXFP8(x) . W) over the E4M3 weights w13_8
    [2I, H] (gate rows first); x [R, H] fp64 values."""
    I = w13_8.shape[0] // 2
    xq = _mx_value(x)
    g = float(tscale) * (xq @ w13_8[:I].T)
    u = float(tscale) * (xq @ w13_8[I:].T)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def swiglu_ffn_w4a8(x, w13_8, ts13, w2_8, ts2) -> np.ndarray:
    """y = ts2 * MXFP8(h) . W2_8 with h = BF16(swiglu_hidden_w4a8(x)); y rounded to BF16."""
    h = bf16_round(swiglu_hidden_w4a8(x, w13_8, ts13))
    return bf16_round(float(ts2) * (_mx_value(h) @ w2_8.T))


def layer_w4a8(inp, tokens=None, logits=None):
    """The whole layer with the W4A8 FFN (reading R18) for the routed experts and the
    shared expert; routing, combine and norm as in ``layer``. Returns the same dict
    (without the plan), plus the BF16 h of every (token, slot) ("h", [T, k, I]) and of
    the shared expert ("h_shared")."""
    wl = inp.w
    T = inp.x.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    if logits is None:
        logits = (np.asarray(inp.logits, dtype=np.float64)[tok] if inp.logits is not None
                  else router_logits(np.asarray(inp.x)[tok], inp.w_router))
    idx, w = route(logits, wl.k)
    x = bf16_value(np.asarray(inp.x)[tok])
    y = np.zeros((len(tok), wl.k, x.shape[1]), dtype=np.float64)
    h = np.zeros((len(tok), wl.k, wl.I), dtype=np.float64)
    for e in np.unique(idx):
        rr, jj = np.nonzero(idx == e)
        W13 = dequant_e4m3(inp.w13.packed[e], inp.w13.scales[e])
        W2 = dequant_e4m3(inp.w2.packed[e], inp.w2.scales[e])
        h[rr, jj] = bf16_round(swiglu_hidden_w4a8(x[rr], W13, inp.w13.tscale[e]))
        y[rr, jj] = swiglu_ffn_w4a8(x[rr], W13, inp.w13.tscale[e], W2, inp.w2.tscale[e])
    shared = h_shared = None
    if getattr(inp, "shared13", None) is not None:
        S13 = dequant_e4m3(inp.shared13.packed[0], inp.shared13.scales[0])
        S2 = dequant_e4m3(inp.shared2.packed[0], inp.shared2.scales[0])
        h_shared = bf16_round(swiglu_hidden_w4a8(x, S13, inp.shared13.tscale[0]))
        shared = swiglu_ffn_w4a8(x, S13, inp.shared13.tscale[0], S2, inp.shared2.tscale[0])
    o, n = combine_norm(y, w, np.asarray(inp.residual)[tok], inp.gamma, wl.eps, shared)
    return {"logits": logits, "idx": idx, "w": w, "y": y, "o": o, "n": n, "tokens": tok, "shared": shared,
            "h": h, "h_shared": h_shared}
