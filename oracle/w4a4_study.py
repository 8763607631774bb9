"""Accuracy study of a W4A4 prefill form for the native FP4 MFMA (test infrastructure,
CPU only; no GPU path computes this form).

The FP8 prompt-matmul option of the Qiita TensorFold 1.1.x article ("Why it still does
not reach 0.6.6") has a further step down on gfx950: the block-scaled MFMA also takes
E2M1 operands, at twice the FP8 rate. The PR804 article's NVFP4 section tells W4A16
(4-bit weights, 16-bit activations) apart from 4-bit compute. What the FP4 MFMA needs,
and what it would cost in accuracy, is read here as follows (reading R19, a study, not a
supported form):

* activations in blocks of 32 consecutive values along K, each with a power-of-two
  scale 2^e, e the smallest integer for which the block's largest magnitude times 2^-e
  is at most 6 (the largest E2M1 value; e = 0 for an all-zero block), the scaled values
  rounded to E2M1 (nearest, ties to even);
* weights: the MFMA's operand scale is one power of two per 32 weights along K, while
  the checkpoint has one E4M3 scale per 16, so each block of 32 dequantised weights
  (code * E4M3 scale, exact) is requantised the same way as the activations;
* sums and the rest of the FFN as in W4A16 (h BF16, requantised for the down GEMM).

``study()`` reports the error of the expert outputs of the W4A8 form (reading R18,
``oracle.swiglu_ffn_w4a8``) and of this form against the W4A16 oracle on seeded inputs
of a workload.
"""
from __future__ import annotations

import numpy as np

from . import (bf16_round, bf16_value, dequant, dequant_e4m3, route, swiglu_ffn, swiglu_ffn_w4a8)

E2M1_MAX = 6.0


def e2m1_round(v: np.ndarray) -> np.ndarray:
    """fp64 -> the nearest E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives), ties
    to even, saturating at +-6. The spacing is 0.5 below 2, 1 in [2, 4) and 2 from 4
    on; |v| is divided by its spacing and rounded to an integer (np.rint: half to
    even)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.rint(a / step) * step
    return np.copysign(np.minimum(r, E2M1_MAX), v)


def mxfp4_quantize(x: np.ndarray, block: int = 32):
    """x [..., K] -> (q, e): q fp64 E2M1 values [..., K], e int [..., K/block], with
    x ~ q * 2^e. e is the smallest integer with max|block| * 2^-e <= 6: with
    max|block| = m * 2^E (1 <= m < 2), e = E - 2 when m <= 1.5 and E - 1 otherwise;
    0 for an all-zero block."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % block:
        raise ValueError(f"K={K} is not a multiple of {block}")
    xb = x.reshape(x.shape[:-1] + (K // block, block))
    amax = np.max(np.abs(xb), axis=-1)
    f, E = np.frexp(amax)              # amax = (2f) * 2^(E-1)
    e = np.where(2.0 * f <= 1.5, E - 1 - 2, E - 1 - 1)
    e = np.where(amax == 0, 0, e).astype(np.int64)
    q = e2m1_round(np.ldexp(xb, -e[..., None]))
    return q.reshape(x.shape), e


def mx4_value(x: np.ndarray, block: int = 32) -> np.ndarray:
    q, e = mxfp4_quantize(x, block)
    return (q.reshape(e.shape + (block,)) * np.exp2(e)[..., None]).reshape(q.shape)


def swiglu_ffn_w4a4(x, w13_4, ts13, w2_4, ts2) -> np.ndarray:
    """y = ts2 * MX4(h) . W2_4 with h = BF16(silu(g) * u), g, u = ts13 * MX4(x) . W13_4;
    W13_4 and W2_4 the requantised weights (mx4_value of the dequantised ones)."""
    I = w13_4.shape[0] // 2
    xq = mx4_value(x)
    g = float(ts13) * (xq @ w13_4[:I].T)
    u = float(ts13) * (xq @ w13_4[I:].T)
    with np.errstate(over="ignore"):
        h = bf16_round(g / (1.0 + np.exp(-g)) * u)
    return bf16_round(float(ts2) * (mx4_value(h) @ w2_4.T))


def swiglu_ffn_mixed(x, w13, ts13, w2, ts2, act) -> np.ndarray:
    """The FFN with the given weights (already in their final form) and `act` applied to
    its two activation inputs (x and the BF16 h): for splitting the W4A4 error between
    the activations (exact weights, act = mx4_value) and the weights (requantised
    weights, act = identity)."""
    I = w13.shape[0] // 2
    xq = act(x)
    g = float(ts13) * (xq @ w13[:I].T)
    u = float(ts13) * (xq @ w13[I:].T)
    with np.errstate(over="ignore"):
        h = bf16_round(g / (1.0 + np.exp(-g)) * u)
    return bf16_round(float(ts2) * (act(h) @ w2.T))


def study(inp, tokens: np.ndarray, experts: int = 8):
    """Relative rms and max errors of the expert outputs y against the W4A16 oracle, over
    the routed rows of `tokens` that go to the first `experts` experts they touch, for
    the W4A8 form, the W4A4 form, and W4A4's two halves alone (FP4 activations with the
    exact weights; the requantised weights with BF16 activations). Returns a dict of
    {form: (rel_rms, rel_max)}."""
    wl = inp.w
    L = np.asarray(inp.logits, dtype=np.float64)[tokens]
    idx, _ = route(L, wl.k)
    x = bf16_value(np.asarray(inp.x)[tokens])
    ref, f8, f4, fa, fw = [], [], [], [], []
    for e in np.unique(idx)[:experts]:
        rr, _ = np.nonzero(idx == e)
        W13 = dequant(inp.w13.packed[e], inp.w13.scales[e], inp.w13.tscale[e])
        W2 = dequant(inp.w2.packed[e], inp.w2.scales[e], inp.w2.tscale[e])
        ref.append(swiglu_ffn(x[rr], W13, W2))
        W13_8 = dequant_e4m3(inp.w13.packed[e], inp.w13.scales[e])
        W2_8 = dequant_e4m3(inp.w2.packed[e], inp.w2.scales[e])
        f8.append(swiglu_ffn_w4a8(x[rr], W13_8, inp.w13.tscale[e], W2_8, inp.w2.tscale[e]))
        W13_4 = mx4_value(dequant(inp.w13.packed[e], inp.w13.scales[e], 1.0))
        W2_4 = mx4_value(dequant(inp.w2.packed[e], inp.w2.scales[e], 1.0))
        f4.append(swiglu_ffn_w4a4(x[rr], W13_4, inp.w13.tscale[e], W2_4, inp.w2.tscale[e]))
        ident = lambda v: v
        fa.append(swiglu_ffn_mixed(x[rr], W13 / float(inp.w13.tscale[e]), inp.w13.tscale[e],
                                   W2 / float(inp.w2.tscale[e]), inp.w2.tscale[e], mx4_value))
        fw.append(swiglu_ffn_mixed(x[rr], W13_4, inp.w13.tscale[e], W2_4, inp.w2.tscale[e], ident))
    ref = np.concatenate(ref)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    out = {}
    for name, got in (("w4a8", np.concatenate(f8)), ("w4a4", np.concatenate(f4)),
                      ("fp4 activations only", np.concatenate(fa)), ("requantised weights only", np.concatenate(fw))):
        d = got - ref
        out[name] = (float(np.sqrt(np.mean(d ** 2))) / rms, float(np.max(np.abs(d))) / rms)
    return out
