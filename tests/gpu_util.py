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


def upload_weights(inp: wl.LayerInputs):
    w13 = B.DeviceW4.from_host(inp.w13)
    w2 = B.DeviceW4.from_host(inp.w2)
    s13 = B.DeviceW4.from_host(inp.shared13) if inp.shared13 is not None else None
    s2 = B.DeviceW4.from_host(inp.shared2) if inp.shared2 is not None else None
    wr = to_dev(inp.w_router) if inp.w_router is not None else None
    return w13, w2, s13, s2, wr


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
