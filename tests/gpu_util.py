"""Helpers for the GPU parity tests: upload seeded inputs, run the C ABI through the
binding, and condition computed-logit inputs on a top-k margin (test side only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from bit_moe_expert_amd import binding as B
from bit_moe_expert_amd import workloads as wl


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_value(to_host_bits(t))


def top_margins_ok(L: np.ndarray, k: int, margin: float) -> np.ndarray:
    m = min(k + 1, L.shape[1])
    top = -np.sort(-L, axis=1)[:, :m]
    return np.all(top[:, :-1] - top[:, 1:] >= margin, axis=1)


def condition_router_margin(inp: wl.LayerInputs, margin: float = 1e-3, attempts: int = 64) -> int:
    """Redraw activation rows until the fp64 router logits of every token have
    consecutive gaps >= margin among their top k+1 (so an FP32 router decides the
    same experts). Returns the number of redrawn rows."""
    redrawn = 0
    for attempt in range(attempts):
        L = oracle.router_logits(inp.x, inp.w_router)
        bad = np.flatnonzero(~top_margins_ok(L, inp.w.k, margin))
        if bad.size == 0:
            return redrawn
        redrawn += bad.size
        wl.redraw_x_rows(inp, bad, attempt)
    raise RuntimeError("router margin conditioning did not converge")


class GpuLayer:
    """One layer call's inputs and outputs resident on the GPU."""

    def __init__(self, inp: wl.LayerInputs, weights=None):
        w = inp.w
        T = inp.T
        self.inp = inp
        self.shape = B.make_shape(T, w.H, w.E, w.k, w.I, w.n_shared, w.eps)
        self.x = to_dev(inp.x)
        self.residual = to_dev(inp.residual)
        self.gamma = to_dev(inp.gamma)
        if weights is None:
            weights = upload_weights(inp)
        self.w13, self.w2, self.shared13, self.shared2, self.w_router = weights
        if inp.logits is not None:
            self.logits = to_dev(inp.logits)
        else:
            self.logits = torch.empty((T, w.E), dtype=torch.float32, device="cuda")
        self.topk_idx = torch.full((T, w.k), -1, dtype=torch.int32, device="cuda")
        self.topk_w = torch.zeros((T, w.k), dtype=torch.float32, device="cuda")
        self.res_out = torch.zeros((T, w.H), dtype=torch.int16, device="cuda")
        self.norm_out = torch.zeros((T, w.H), dtype=torch.int16, device="cuda")
        self.ws = torch.empty(max(1, B.moe4_layer_workspace_bytes(self.shape)), dtype=torch.uint8,
                              device="cuda")

    def run(self, stream=None, side_stream=None):
        B.moe4_layer(self.shape, self.x, self.w_router, self.logits, self.w13, self.w2,
                     self.shared13, self.shared2, self.residual, self.gamma, self.topk_idx,
                     self.topk_w, self.res_out, self.norm_out, self.ws, stream=stream,
                     side_stream=side_stream)

    def host(self):
        torch.cuda.synchronize()
        return {
            "idx": self.topk_idx.cpu().numpy(),
            "w": self.topk_w.cpu().numpy().astype(np.float64),
            "logits": self.logits.cpu().numpy().astype(np.float64),
            "o": bf16_f64(self.res_out),
            "n": bf16_f64(self.norm_out),
            "o_bits": to_host_bits(self.res_out),
            "n_bits": to_host_bits(self.norm_out),
        }


def upload_weights(inp: wl.LayerInputs, layout: str = "tiled"):
    w13 = B.DeviceW4.from_host(inp.w13, layout=layout)
    w2 = B.DeviceW4.from_host(inp.w2, layout=layout)
    s13 = B.DeviceW4.from_host(inp.shared13, layout=layout) if inp.shared13 is not None else None
    s2 = B.DeviceW4.from_host(inp.shared2, layout=layout) if inp.shared2 is not None else None
    wr = to_dev(inp.w_router) if inp.w_router is not None else None
    return w13, w2, s13, s2, wr


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """The BF16 spacing at |v| (8 significant bits: 2^(floor(log2|v|) - 7))."""
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(np.asarray(v, np.float64)), 1e-300))) - 7)


LAYER_TOL = 2e-2


def layer_excess(got_o: np.ndarray, got_n: np.ndarray, ref: dict, gamma_bits: np.ndarray, eps: float,
                 sel=slice(None)):
    """How far the layer outputs o and n exceed the bar, as a fraction of rms(ref).

    The bar: max |gpu - ref| <= 2e-2 * rms(ref) over the tensor, for the computation
    error beyond BF16 storage. Two BF16 roundings are not computation error: the GPU's
    output is a BF16 value (at best half a BF16 ulp from the exact one), and each expert
    output y (BF16 on both sides) may round to the neighbouring value when the GPU's
    FP32 sum and the oracle's fp64 sum straddle a rounding boundary (one ulp of y,
    weighted by its routing weight; the shared expert's output with weight 1). So each
    element may be off by 2e-2 * rms(ref) + ulp(gpu) / 2 + sum_j w_j ulp(y_j) (+ ulp(s)),
    the y part carried through the norm as gamma / rms(o_t) for n. Returns
    (excess_o, excess_n, raw_o, raw_n): excess = max(|err| - slack) / rms(ref) (the bar
    holds iff it is <= 2e-2) and raw = max |err| / rms(ref) without the slack."""
    ro, rn = ref["o"][sel], ref["n"][sel]
    ydev = np.einsum("tj,tjh->th", ref["w"][sel], bf16_ulp(ref["y"][sel]))
    if ref.get("shared") is not None:
        ydev = ydev + bf16_ulp(ref["shared"][sel])
    gam = oracle.bf16_value(gamma_bits)[None, :]
    rms_t = np.sqrt(np.mean(ro * ro, axis=1, keepdims=True) + eps)
    slack_o = 0.5 * bf16_ulp(got_o) + ydev
    slack_n = 0.5 * bf16_ulp(got_n) + gam / rms_t * ydev
    rms_o, rms_n = float(np.sqrt(np.mean(ro * ro))), float(np.sqrt(np.mean(rn * rn)))
    eo, en = np.abs(got_o - ro), np.abs(got_n - rn)
    return (float(np.max(eo - slack_o)) / rms_o, float(np.max(en - slack_n)) / rms_n,
            float(np.max(eo)) / rms_o, float(np.max(en)) / rms_n)


def assert_layer_close(got_o, got_n, ref, gamma_bits, eps, what="layer", sel=slice(None)):
    ex_o, ex_n, raw_o, raw_n = layer_excess(got_o, got_n, ref, gamma_bits, eps, sel)
    print(f"  {what}: error beyond BF16 storage o={ex_o:.2e} n={ex_n:.2e} of rms "
          f"(raw max|err|/rms o={raw_o:.2e} n={raw_n:.2e})", flush=True)
    assert ex_o <= LAYER_TOL and ex_n <= LAYER_TOL, f"{what}: o {ex_o:.3e}, n {ex_n:.3e} > {LAYER_TOL}"


def rel_rms_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / rms(ref) over the whole tensor."""
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got - ref)))


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what: str, slack_rms: float = 2.0 ** -12,
                      min_equal: float = 0.9) -> None:
    """BF16 results vs BF16-rounded oracle values: each within one BF16 ulp of the
    reference (the two roundings may fall on either side of a boundary when FP32 and
    fp64 sums differ), plus `slack_rms` * rms(ref) for the FP32 summation and flips
    of upstream BF16 values; most elements bit-equal."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))) - 7)
    bad = np.abs(got - ref) > ulp + slack_rms * rms
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond 1 ulp + slack; worst " \
        f"{float(np.max(np.abs(got - ref) / (ulp + slack_rms * rms))):.2f}x"
    eq = float(np.mean(got == ref))
    assert eq >= min_equal, f"{what}: only {eq:.3f} of elements bit-equal"


# ----------------------------------------------------------------------------
# Layer bar of the FP8 (W4A8) form
# ----------------------------------------------------------------------------
FLIP_SIGMAS = 4.0


def _mx_candidates(h: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """For BF16 h rows [R, I] and per-element allowances delta: the largest change of
    each element's MXFP8 value when h moves anywhere within +-delta (the block scale
    recomputed from the moved block maximum, the value rounded at it). 0 where every
    such h gives the oracle's own code."""
    R, I = h.shape
    hb = h.reshape(R, I // 32, 32)
    db = delta.reshape(R, I // 32, 32)
    _, e0 = oracle.mxfp8_quantize(h)
    amax = np.max(np.abs(hb), axis=-1)
    # block exponents the moved maximum can select (the decision is monotone in amax)
    amax_d = np.max(db, axis=-1)
    _, e_lo = oracle.mxfp8_quantize(np.repeat(np.maximum(amax - amax_d, 0.0), 32, axis=-1).reshape(R, I))
    _, e_hi = oracle.mxfp8_quantize(np.repeat(amax + amax_d, 32, axis=-1).reshape(R, I))
    q0 = oracle.e4m3_round(np.ldexp(hb, -e0[..., None])) * np.exp2(e0)[..., None]
    worst = np.zeros_like(hb)
    for e in (e_lo, e0, e_hi):
        sc = np.exp2(e)[..., None]
        for d in (-db, db):
            q = oracle.e4m3_round(np.ldexp(hb + d, -e[..., None])) * sc
            worst = np.maximum(worst, np.abs(q - q0))
    return worst.reshape(R, I)


def w4a8_flip_slack(ref: dict, inp, h_bar_rms: float = 2.0 ** -12):
    """Per-element slack on y (and hence on o) for h codes the GPU may legitimately
    choose differently: the GPU's BF16 h is within one BF16 ulp plus h_bar_rms of the
    row's rms of the oracle's (the h step bar), and an E4M3 code of h changes (by a
    whole E4M3 step, 1/8 of the value) whenever h crosses a rounding boundary, however
    small the move. So each h element that lies within that allowance of a boundary
    may flip, and y[n] may move by W2[n, i] * (its change) for each. Flips of
    different elements are independent, with signs set by W2, so the slack is
    FLIP_SIGMAS times the root of the sum of squares of those terms over the elements
    that can flip (the terms of the elements that do flip are a subset); the routing
    weights combine the k experts' slacks the same way (the shared expert with weight
    1). Returns [T, H] for o."""
    idx, w = ref["idx"], ref["w"]
    H = ref["o"].shape[1]
    var = np.zeros((idx.shape[0], H))

    def rss(h_rows, m2, e):
        rms = np.sqrt(np.mean(h_rows ** 2, axis=1, keepdims=True))
        delta = bf16_ulp(h_rows) + h_bar_rms * rms
        dq = _mx_candidates(h_rows, delta)
        w2sq = oracle.dequant_e4m3(m2.packed[e], m2.scales[e]) ** 2
        return float(m2.tscale[e]) ** 2 * ((dq ** 2) @ w2sq.T)   # [rows, H]

    for e in np.unique(idx):
        rr, jj = np.nonzero(idx == e)
        var[rr] += (w[rr, jj] ** 2)[:, None] * rss(ref["h"][rr, jj], inp.w2, e)
    if ref.get("h_shared") is not None:
        var += rss(ref["h_shared"], inp.shared2, 0)
    return FLIP_SIGMAS * np.sqrt(var)


def assert_layer_close_w4a8(got_o, got_n, ref, inp, what="w4a8 layer", sel=slice(None)):
    """The layer bar of the FP8 form. The W4A16 bar (max |err| <= 2e-2 * rms(ref)
    beyond BF16 storage) cannot hold as it stands: requantising h to E4M3 turns a
    one-ulp BF16 difference into a whole E4M3 step wherever h sits at a rounding
    boundary (measured with the oracle alone: 1-ulp moves of 10 % of h elements move y
    by up to 16 % of its rms). So:
      * each token's rms error is at most 2e-2 * rms(ref) plus the rms over the row of
        one sigma of the flip bound (w4a8_flip_slack / FLIP_SIGMAS);
      * each element's error is at most the W4A16 bar plus w4a8_flip_slack.
    Checked on the CPU with the oracle alone: 1-ulp moves of 10 % of its h pass, and
    one h block of one row at twice its scale fails."""
    ro, rn = ref["o"][sel], ref["n"][sel]
    rms_o, rms_n = float(np.sqrt(np.mean(ro * ro))), float(np.sqrt(np.mean(rn * rn)))
    flip = w4a8_flip_slack(ref, inp)[sel]
    gam = oracle.bf16_value(inp.gamma)[None, :]
    rms_t = np.sqrt(np.mean(ro * ro, axis=1, keepdims=True) + inp.w.eps)
    sig_o = np.sqrt(np.mean((flip / FLIP_SIGMAS) ** 2, axis=1)) / rms_o
    sig_n = np.sqrt(np.mean((gam / rms_t * flip / FLIP_SIGMAS) ** 2, axis=1)) / rms_n
    row_o = np.sqrt(np.mean((got_o - ro) ** 2, axis=1)) / rms_o - sig_o
    row_n = np.sqrt(np.mean((got_n - rn) ** 2, axis=1)) / rms_n - sig_n
    ydev = np.einsum("tj,tjh->th", ref["w"][sel], bf16_ulp(ref["y"][sel]))
    if ref.get("shared") is not None:
        ydev = ydev + bf16_ulp(ref["shared"][sel])
    slack_o = 0.5 * bf16_ulp(got_o) + ydev + flip
    slack_n = 0.5 * bf16_ulp(got_n) + gam / rms_t * (ydev + flip)
    ex_o = float(np.max(np.abs(got_o - ro) - slack_o)) / rms_o
    ex_n = float(np.max(np.abs(got_n - rn) - slack_n)) / rms_n
    print(f"  {what}: worst token rms error beyond the flip sigma o={row_o.max():.2e} n={row_n.max():.2e} of rms; "
          f"element error beyond "
          f"storage + flip slack o={ex_o:.2e} n={ex_n:.2e} (flip slack mean {float(np.mean(flip)) / rms_o:.2e} "
          f"of rms, raw max|err|/rms o={float(np.max(np.abs(got_o - ro))) / rms_o:.2e})", flush=True)
    assert row_o.max() <= LAYER_TOL and row_n.max() <= LAYER_TOL, \
        f"{what}: token rms error o {row_o.max():.3e}, n {row_n.max():.3e} > {LAYER_TOL}"
    assert ex_o <= LAYER_TOL and ex_n <= LAYER_TOL, f"{what}: o {ex_o:.3e}, n {ex_n:.3e} > {LAYER_TOL}"
