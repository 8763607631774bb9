"""Seeded synthetic inputs for the W4A16 MoE layer.

This module draws inputs and stores them in the layer's storage formats. It holds
none of the layer's arithmetic (no dequantisation, routing, matmul or norm), so the
fp64 oracle and the HIP path can both take their inputs from here without sharing
any of the computation they are compared on.

Storage formats (the checkpoint-style NVFP4 layout, read as is):
  * BF16 tensors are ``uint16`` bit patterns.
  * FP8 E4M3 scales (OCP E4M3FN) are ``uint8`` codes.
  * 4-bit E2M1 weights are packed two per byte along K: element ``2j`` in the low
    nibble, element ``2j+1`` in the high nibble.
  * One E4M3 scale covers 16 consecutive weights along K.
  * One FP32 tensor scale per expert matrix.

Weight matrices, per expert ``e``:
  * W13: ``N = 2I`` rows (rows ``0..I-1`` gate, ``I..2I-1`` up), ``K = H``.
  * W2:  ``N = H`` rows, ``K = I``.

Draw recipe (each tensor has its own child of ``SeedSequence(seed)``, taken in a
fixed order, so changing one tensor's shape does not move the others):
  * activations ``x`` and ``residual``: N(0,1) rounded to BF16;
  * RMSNorm gamma: U(0.5, 1.5) rounded to BF16;
  * weight codes: uniform over the 16 E2M1 codes (uniform random bytes);
  * block scales: ``2**u`` with ``u ~ U(-4, 2)``, rounded to E4M3;
  * tensor scales: 1.0;
  * router: either FP32 logits drawn directly (N(0,1) i.i.d. = uniform routing, or
    ``log p_e + Gumbel`` with Zipf popularity ``p_e ~ (e+1)^-s``), or BF16 router
    weights N(0, 0.02) from which the layer computes the logits itself.

The tiny workload asks for a top-k margin of at least 1e-3 on its given logits:
rows whose top k+1 logits (sorted) have a consecutive gap below that are re-drawn
from a further child stream until they pass.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np
import torch


# ----------------------------------------------------------------------------
# Workload shapes (the pages' MoE layers at the sizes this library is measured on)
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    T: int               # tokens per layer call
    H: int               # hidden size
    E: int               # routed experts
    k: int               # experts per token
    I: int               # expert FFN intermediate size
    routing: str         # "normal" | "zipf" | "router"
    n_shared: int = 0    # always-on shared experts (0 or 1)
    chunks: int = 1      # layer calls per workload (long prefill is chunked)
    margin: float = 0.0  # enforced top-k margin on given logits
    zipf_s: float = 1.1
    router_std: float = 0.02
    eps: float = 1e-6

    @property
    def rows(self) -> int:
        """Rows through the expert FFN per call: routed pairs plus shared rows."""
        return self.T * self.k + self.T * self.n_shared


WORKLOADS: Dict[str, Workload] = {
    # tiny layer, latency only; given N(0,1) logits with margin >= 1e-3
    "tiny": Workload("tiny", T=16, H=256, E=8, k=2, I=512, routing="normal", margin=1e-3),
    # decode: router logits computed from BF16 router weights N(0, 0.02)
    "decode_t1": Workload("decode_t1", T=1, H=2048, E=128, k=8, I=768, routing="router"),
    "decode_t8": Workload("decode_t8", T=8, H=2048, E=128, k=8, I=768, routing="router"),
    # batched decode: uniform routing (i.i.d. N(0,1) logits)
    "batched_t64": Workload("batched_t64", T=64, H=4096, E=256, k=8, I=2048, routing="normal"),
    "batched_t256": Workload("batched_t256", T=256, H=4096, E=256, k=8, I=2048, routing="normal"),
    # prefill: Zipf(1.1) expert popularity
    "prefill": Workload("prefill", T=8192, H=4096, E=128, k=8, I=1536, routing="zipf"),
    # long prefill: 32768 tokens as 4 chunks of 8192, plus one shared expert
    "long_prefill": Workload("long_prefill", T=8192, H=6144, E=160, k=8, I=2048,
                             routing="zipf", n_shared=1, chunks=4),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (for reduced-size tests)."""
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


# ----------------------------------------------------------------------------
# Storage-format conversions (library routines; no layer arithmetic)
# ----------------------------------------------------------------------------
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float values to BF16 (torch's round-to-nearest-even) and return the bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """Round float values to OCP FP8 E4M3FN (torch.float8_e4m3fn) and return the codes."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------------------
# Drawing helpers
# ----------------------------------------------------------------------------
_CHUNK = 1 << 24


def _bf16_normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = to_bf16_bits(rng.standard_normal(e - s) * std)
    return out.reshape(shape)


def _random_codes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


def _log_uniform_e4m3(rng: np.random.Generator, shape, lo: float = -4.0, hi: float = 2.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        u = rng.random(e - s) * (hi - lo) + lo
        out[s:e] = to_e4m3_codes(np.exp2(u))
    return out.reshape(shape)


@dataclass
class W4Matrix:
    """One grouped 4-bit weight tensor: E experts, N rows, K columns."""
    packed: np.ndarray   # uint8 [E, N, K/2]
    scales: np.ndarray   # uint8 [E, N, K/16] (E4M3 codes)
    tscale: np.ndarray   # float32 [E]

    @property
    def shape(self):
        E, N, K2 = self.packed.shape
        return E, N, 2 * K2


def draw_w4(ss: np.random.SeedSequence, E: int, N: int, K: int) -> W4Matrix:
    """Uniform E2M1 codes, log-uniform E4M3 block scales, unit tensor scales."""
    assert K % 16 == 0
    s_codes, s_scales = ss.spawn(2)
    return W4Matrix(
        packed=_random_codes(np.random.default_rng(s_codes), (E, N, K // 2)),
        scales=_log_uniform_e4m3(np.random.default_rng(s_scales), (E, N, K // 16)),
        tscale=np.ones(E, dtype=np.float32),
    )


def _margin_ok(rows: np.ndarray, k: int, margin: float) -> np.ndarray:
    """Per row: do the top k+1 values, sorted, have every consecutive gap >= margin?"""
    m = min(k + 1, rows.shape[1])
    top = -np.sort(-rows.astype(np.float64), axis=1)[:, :m]
    if m < 2:
        return np.ones(rows.shape[0], dtype=bool)
    return np.all(top[:, :-1] - top[:, 1:] >= margin, axis=1)


def _draw_logits(ss: np.random.SeedSequence, w: Workload, T: int) -> np.ndarray:
    s_main, s_redraw = ss.spawn(2)
    rng = np.random.default_rng(s_main)
    if w.routing == "normal":
        logits = rng.standard_normal((T, w.E)).astype(np.float32)
    elif w.routing == "zipf":
        ranks = np.arange(1, w.E + 1, dtype=np.float64)
        p = ranks ** (-w.zipf_s)
        p /= p.sum()
        u = rng.random((T, w.E))
        u = np.clip(u, np.finfo(np.float64).tiny, None)
        gumbel = -np.log(-np.log(u))
        logits = (np.log(p)[None, :] + gumbel).astype(np.float32)
    else:
        raise ValueError(w.routing)
    if w.margin > 0:
        rr = np.random.default_rng(s_redraw)
        bad = np.flatnonzero(~_margin_ok(logits, w.k, w.margin))
        while bad.size:
            logits[bad] = rr.standard_normal((bad.size, w.E)).astype(np.float32)
            bad = bad[~_margin_ok(logits[bad], w.k, w.margin)]
    return logits


@dataclass
class LayerInputs:
    """Everything one MoE layer call consumes, in storage formats."""
    w: Workload
    x: np.ndarray                 # uint16 [T, H]
    residual: np.ndarray          # uint16 [T, H]
    gamma: np.ndarray             # uint16 [H]
    w13: W4Matrix                 # [E, 2I, H]
    w2: W4Matrix                  # [E, H, I]
    logits: Optional[np.ndarray]  # float32 [T, E] when given
    w_router: Optional[np.ndarray]  # uint16 [E, H] when the layer computes logits
    shared13: Optional[W4Matrix] = None  # [1, 2I, H]
    shared2: Optional[W4Matrix] = None   # [1, H, I]
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.x.shape[0]


def make_inputs(w: Workload, seed: int = 0, chunk: int = 0, T: Optional[int] = None,
                weights_from: Optional["LayerInputs"] = None) -> LayerInputs:
    """Inputs of one layer call of workload ``w``.

    ``chunk`` selects the token chunk of a chunked workload: weights, router and
    gamma are the same for every chunk; activations, residual and logits differ.
    ``T`` overrides the token count (for reduced-size tests). ``weights_from`` (the
    inputs of another chunk of the same workload and seed) reuses its weights, router
    and gamma instead of drawing them again: the draws would be the same.
    """
    T = w.T if T is None else T
    root = np.random.SeedSequence(seed)
    (s_weights, s_chunks) = root.spawn(2)
    s_w13, s_w2, s_gamma, s_router, s_sh13, s_sh2 = s_weights.spawn(6)
    s_tok = np.random.SeedSequence([seed, 7919, chunk])
    s_x, s_res, s_logits = s_tok.spawn(3)

    x = _bf16_normal(np.random.default_rng(s_x), (T, w.H))
    residual = _bf16_normal(np.random.default_rng(s_res), (T, w.H))
    logits = None
    if w.routing != "router":
        logits = _draw_logits(s_logits, w, T)
    if weights_from is not None:
        if weights_from.w != w or weights_from.seed != seed:
            raise ValueError("weights_from must be inputs of the same workload and seed")
        b = weights_from
        return LayerInputs(w=w, x=x, residual=residual, gamma=b.gamma, w13=b.w13, w2=b.w2,
                           logits=logits, w_router=b.w_router, shared13=b.shared13,
                           shared2=b.shared2, seed=seed)
    gamma_rng = np.random.default_rng(s_gamma)
    gamma = to_bf16_bits(gamma_rng.uniform(0.5, 1.5, w.H))
    w13 = draw_w4(s_w13, w.E, 2 * w.I, w.H)
    w2 = draw_w4(s_w2, w.E, w.H, w.I)
    w_router = None
    if w.routing == "router":
        w_router = _bf16_normal(np.random.default_rng(s_router), (w.E, w.H), std=w.router_std)
    shared13 = shared2 = None
    if w.n_shared:
        shared13 = draw_w4(s_sh13, w.n_shared, 2 * w.I, w.H)
        shared2 = draw_w4(s_sh2, w.n_shared, w.H, w.I)
    return LayerInputs(w=w, x=x, residual=residual, gamma=gamma, w13=w13, w2=w2,
                       logits=logits, w_router=w_router, shared13=shared13,
                       shared2=shared2, seed=seed)


def redraw_x_rows(inp: LayerInputs, rows: np.ndarray, attempt: int) -> None:
    """Replace activation rows ``rows`` with fresh BF16 N(0,1) draws (in place).

    Used by callers that condition computed-logit inputs on a top-k margin; the
    stream depends only on (seed, attempt), never on the values being replaced.
    """
    rng = np.random.default_rng(np.random.SeedSequence([inp.seed, 104729, attempt]))
    inp.x[rows] = _bf16_normal(rng, (len(rows), inp.x.shape[1]))
