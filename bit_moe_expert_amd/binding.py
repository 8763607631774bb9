"""Thin torch binding over the libmoe4 C ABI: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch tensors
that already live on the GPU (BF16 tensors may be ``torch.bfloat16`` or the raw
``uint16``/``int16`` bits). Work is enqueued on the current torch stream (or the
one given); nothing is synchronised or computed here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import Shape, W4, check

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)
_F16_LIKE = (torch.float16, torch.int16, torch.uint16)


def _ptr(t: Optional[torch.Tensor], name: str, dtypes=None, numel: Optional[int] = None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_shape(T: int, H: int, E: int, k: int, I: int, n_shared: int = 0, eps: float = 1e-6) -> Shape:
    return Shape(T, H, E, k, I, n_shared, eps)


def moe4_prepack_w4(G: int, N: int, K: int, codes, scales, tcodes, tscales, stream=None) -> None:
    n = G * N * K
    check(_lib.load().moe4_prepack_w4(
        G, N, K, _ptr(codes, "codes", (torch.uint8,), n // 2), _ptr(scales, "scales", (torch.uint8,), n // 16),
        _ptr(tcodes, "tcodes", (torch.uint8,), n // 2), _ptr(tscales, "tscales", (torch.uint8,), n // 16),
        _stream(stream)))


@dataclass
class DeviceW4:
    """A grouped 4-bit weight tensor resident on the GPU, in the tiled layout (the
    canonical bytes re-laid out once by moe4_prepack_w4, faster to stream) or in the
    canonical (checkpoint) layout as uploaded."""
    packed: torch.Tensor   # uint8 [G, N, K/2] bytes
    scales: torch.Tensor   # uint8 [G, N, K/16] bytes
    tscale: torch.Tensor   # float32 [G]
    layout: int = _lib.MOE4_W4_TILED

    @classmethod
    def from_host(cls, w, device="cuda", layout: str = "tiled") -> "DeviceW4":
        """Upload canonical host weights (packed [G,N,K/2], scales [G,N,K/16]); with
        layout="tiled" re-lay them out on the GPU, with "canonical" keep them as they are."""
        G, N, K2 = w.packed.shape
        codes = torch.from_numpy(w.packed).to(device)
        scales = torch.from_numpy(w.scales).to(device)
        tscale = torch.from_numpy(w.tscale).to(device)
        if layout == "canonical":
            return cls(codes, scales, tscale, _lib.MOE4_W4_CANONICAL)
        if layout != "tiled":
            raise ValueError(f"layout must be 'tiled' or 'canonical', not {layout!r}")
        tcodes = torch.empty_like(codes)
        tscales = torch.empty_like(scales)
        moe4_prepack_w4(G, N, 2 * K2, codes, scales, tcodes, tscales)
        torch.cuda.current_stream().synchronize()
        del codes, scales
        return cls(tcodes, tscales, tscale, _lib.MOE4_W4_TILED)

    def clone(self) -> "DeviceW4":
        return DeviceW4(self.packed.clone(), self.scales.clone(), self.tscale.clone(), self.layout)

    def desc(self) -> W4:
        return W4(_ptr(self.packed, "packed", (torch.uint8,)),
                  _ptr(self.scales, "scales", (torch.uint8,)),
                  _ptr(self.tscale, "tscale", (torch.float32,)), self.layout)

    @property
    def nbytes(self) -> int:
        return self.packed.numel() + self.scales.numel() + 4 * self.tscale.numel()


def moe4_permute_workspace_bytes(shape: Shape) -> int:
    return int(_lib.load().moe4_permute_workspace_bytes(shape))


def moe4_layer_workspace_bytes(shape: Shape) -> int:
    return int(_lib.load().moe4_layer_workspace_bytes(shape))


def moe4_route(shape: Shape, x, w_router, logits, topk_idx, topk_w, stream=None) -> None:
    T, E, k, H = shape.T, shape.E, shape.k, shape.H
    check(_lib.load().moe4_route(
        shape, _ptr(x, "x", _BF16_LIKE, T * H), _ptr(w_router, "w_router", _BF16_LIKE, E * H),
        _ptr(logits, "logits", (torch.float32,), T * E),
        _ptr(topk_idx, "topk_idx", (torch.int32,), T * k),
        _ptr(topk_w, "topk_w", (torch.float32,), T * k), _stream(stream)))


def moe4_permute(shape: Shape, topk_idx, offsets, perm_src, inv, ws=None, stream=None) -> None:
    n = shape.T * shape.k
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    check(_lib.load().moe4_permute(
        shape, _ptr(topk_idx, "topk_idx", (torch.int32,), n),
        _ptr(offsets, "offsets", (torch.int32,), shape.E + 1),
        _ptr(perm_src, "perm_src", (torch.int32,), n), _ptr(inv, "inv", (torch.int32,), n),
        _ptr(ws, "ws"), ws_bytes, _stream(stream)))


def moe4_expert_ffn(shape: Shape, x, offsets, perm_src, w13: DeviceW4, w2: DeviceW4, h, y,
                    stream=None) -> None:
    rows = shape.T * shape.k if offsets is not None else shape.T
    d13, d2 = w13.desc(), w2.desc()
    check(_lib.load().moe4_expert_ffn(
        shape, _ptr(x, "x", _BF16_LIKE, shape.T * shape.H),
        _ptr(offsets, "offsets", (torch.int32,)), _ptr(perm_src, "perm_src", (torch.int32,)),
        d13, d2, _ptr(h, "h", _BF16_LIKE, rows * shape.I), _ptr(y, "y", _BF16_LIKE, rows * shape.H),
        _stream(stream)))


def moe4_expert_up(shape: Shape, x, offsets, perm_src, w13: DeviceW4, h, stream=None) -> None:
    rows = shape.T * shape.k if offsets is not None else shape.T
    d13 = w13.desc()
    check(_lib.load().moe4_expert_up(
        shape, _ptr(x, "x", _BF16_LIKE, shape.T * shape.H),
        _ptr(offsets, "offsets", (torch.int32,)), _ptr(perm_src, "perm_src", (torch.int32,)),
        d13, _ptr(h, "h", _BF16_LIKE, rows * shape.I), _stream(stream)))


def moe4_act_f16(x, x16, xexp, stream=None) -> None:
    """FP16 rows of BF16 x [rows][K], each scaled by its own power of two: x16
    [rows][K] (float16 or 16-bit storage), xexp int32 [rows]."""
    rows, K = x.shape
    check(_lib.load().moe4_act_f16(
        rows, K, _ptr(x, "x", _BF16_LIKE), _ptr(x16, "x16", _F16_LIKE, rows * K),
        _ptr(xexp, "xexp", (torch.int32,), rows), _stream(stream)))


def moe4_expert_up_f16(shape: Shape, x16, xexp, offsets, perm_src, w13: DeviceW4, h, stream=None) -> None:
    rows = shape.T * shape.k if offsets is not None else shape.T
    d13 = w13.desc()
    check(_lib.load().moe4_expert_up_f16(
        shape, _ptr(x16, "x16", _F16_LIKE, shape.T * shape.H), _ptr(xexp, "xexp", (torch.int32,), shape.T),
        _ptr(offsets, "offsets", (torch.int32,)), _ptr(perm_src, "perm_src", (torch.int32,)),
        d13, _ptr(h, "h", _BF16_LIKE, rows * shape.I), _stream(stream)))


def moe4_expert_down(shape: Shape, h, offsets, w2: DeviceW4, y, stream=None) -> None:
    rows = shape.T * shape.k if offsets is not None else shape.T
    d2 = w2.desc()
    check(_lib.load().moe4_expert_down(
        shape, _ptr(h, "h", _BF16_LIKE, rows * shape.I), _ptr(offsets, "offsets", (torch.int32,)),
        d2, _ptr(y, "y", _BF16_LIKE, rows * shape.H), _stream(stream)))


def moe4_combine_norm(shape: Shape, y, inv, topk_w, shared_y, residual, gamma, residual_out,
                      normed_out, stream=None) -> None:
    T, H, k = shape.T, shape.H, shape.k
    check(_lib.load().moe4_combine_norm(
        shape, _ptr(y, "y", _BF16_LIKE, T * k * H), _ptr(inv, "inv", (torch.int32,), T * k),
        _ptr(topk_w, "topk_w", (torch.float32,), T * k),
        _ptr(shared_y, "shared_y", _BF16_LIKE, T * H), _ptr(residual, "residual", _BF16_LIKE, T * H),
        _ptr(gamma, "gamma", _BF16_LIKE, H), _ptr(residual_out, "residual_out", _BF16_LIKE, T * H),
        _ptr(normed_out, "normed_out", _BF16_LIKE, T * H), _stream(stream)))


def moe4_add_rmsnorm(x, residual, gamma, residual_out, normed_out, eps: float = 1e-6,
                     stream=None) -> None:
    """residual_out = x + residual; normed_out = RMSNorm(residual_out) * gamma ([T][H] BF16)."""
    T, H = x.shape
    check(_lib.load().moe4_add_rmsnorm(
        T, H, _ptr(x, "x", _BF16_LIKE, T * H), _ptr(residual, "residual", _BF16_LIKE, T * H),
        _ptr(gamma, "gamma", _BF16_LIKE, H), eps, _ptr(residual_out, "residual_out", _BF16_LIKE, T * H),
        _ptr(normed_out, "normed_out", _BF16_LIKE, T * H), _stream(stream)))


def moe4_group_rmsnorm(x, group: int, gamma, normed_out, eps: float = 1e-6, stream=None) -> None:
    """normed_out = x normalised over each group of ``group`` columns, times gamma."""
    T, H = x.shape
    check(_lib.load().moe4_group_rmsnorm(
        T, H, group, _ptr(x, "x", _BF16_LIKE, T * H), _ptr(gamma, "gamma", _BF16_LIKE, H), eps,
        _ptr(normed_out, "normed_out", _BF16_LIKE, T * H), _stream(stream)))


def moe4_layer(shape: Shape, x, w_router, logits, w13: DeviceW4, w2: DeviceW4,
               shared13: Optional[DeviceW4], shared2: Optional[DeviceW4], residual, gamma,
               topk_idx, topk_w, residual_out, normed_out, ws, stream=None, side_stream=None,
               events=None) -> None:
    """The whole layer. With ``side_stream`` (a torch.cuda.Stream) the routed chain runs
    there while ``stream`` runs the shared expert (moe4_layer_side); ``events`` is a pair
    of torch.cuda.Event for the fork and the join (created on first use if omitted)."""
    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    d13, d2 = w13.desc(), w2.desc()
    s13 = shared13.desc() if shared13 is not None else None
    s2 = shared2.desc() if shared2 is not None else None
    args = (
        shape, _ptr(x, "x", _BF16_LIKE, T * H), _ptr(w_router, "w_router", _BF16_LIKE, E * H),
        _ptr(logits, "logits", (torch.float32,), T * E), d13, d2, s13, s2,
        _ptr(residual, "residual", _BF16_LIKE, T * H), _ptr(gamma, "gamma", _BF16_LIKE, H),
        _ptr(topk_idx, "topk_idx", (torch.int32,), T * k),
        _ptr(topk_w, "topk_w", (torch.float32,), T * k),
        _ptr(residual_out, "residual_out", _BF16_LIKE, T * H),
        _ptr(normed_out, "normed_out", _BF16_LIKE, T * H),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    if side_stream is None:
        check(_lib.load().moe4_layer(*args))
        return
    fork, join = events if events is not None else side_events()
    check(_lib.load().moe4_layer_side(*args, side_stream.cuda_stream, fork.cuda_event, join.cuda_event))


def moe4_layer_noalloc(shape: Shape, x, w_router, logits, w13: DeviceW4, w2: DeviceW4,
                       shared13: Optional[DeviceW4], shared2: Optional[DeviceW4], residual, gamma,
                       topk_idx, topk_w, residual_out, normed_out, stream=None) -> None:
    """The whole layer with the library's static per-GPU scratch instead of a workspace
    (for callers that cannot allocate); shapes beyond its size are rejected."""
    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    d13, d2 = w13.desc(), w2.desc()
    s13 = shared13.desc() if shared13 is not None else None
    s2 = shared2.desc() if shared2 is not None else None
    check(_lib.load().moe4_layer_noalloc(
        shape, _ptr(x, "x", _BF16_LIKE, T * H), _ptr(w_router, "w_router", _BF16_LIKE, E * H),
        _ptr(logits, "logits", (torch.float32,), T * E), d13, d2, s13, s2,
        _ptr(residual, "residual", _BF16_LIKE, T * H), _ptr(gamma, "gamma", _BF16_LIKE, H),
        _ptr(topk_idx, "topk_idx", (torch.int32,), T * k),
        _ptr(topk_w, "topk_w", (torch.float32,), T * k),
        _ptr(residual_out, "residual_out", _BF16_LIKE, T * H),
        _ptr(normed_out, "normed_out", _BF16_LIKE, T * H), _stream(stream)))


def moe4_quant_mxfp8(x, q, e, stream=None) -> None:
    """Block-scaled FP8 of BF16 x [rows][K]: q uint8 [rows][K] E4M3 codes, e uint8
    [rows][K/32] E8M0 scale bytes."""
    rows, K = x.shape
    check(_lib.load().moe4_quant_mxfp8(
        rows, K, _ptr(x, "x", _BF16_LIKE), _ptr(q, "q", (torch.uint8,), rows * K),
        _ptr(e, "e", (torch.uint8,), rows * (K // 32)), _stream(stream)))


def moe4_w4a8_workspace_bytes(shape: Shape) -> int:
    return int(_lib.load().moe4_w4a8_workspace_bytes(shape))


def moe4_expert_ffn_w4a8(shape: Shape, x, offsets, perm_src, w13: DeviceW4, w2: DeviceW4, h, y, ws,
                         stream=None) -> None:
    rows = shape.T * shape.k if offsets is not None else shape.T
    d13, d2 = w13.desc(), w2.desc()
    check(_lib.load().moe4_expert_ffn_w4a8(
        shape, _ptr(x, "x", _BF16_LIKE, shape.T * shape.H),
        _ptr(offsets, "offsets", (torch.int32,)), _ptr(perm_src, "perm_src", (torch.int32,)),
        d13, d2, _ptr(h, "h", _BF16_LIKE, rows * shape.I), _ptr(y, "y", _BF16_LIKE, rows * shape.H),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe4_expert_up_w4a8(shape: Shape, x8, xs, offsets, perm_src, w13: DeviceW4, h, h8, hs,
                        stream=None) -> None:
    rows = shape.T * shape.k if offsets is not None else shape.T
    T, H, I = shape.T, shape.H, shape.I
    d13 = w13.desc()
    check(_lib.load().moe4_expert_up_w4a8(
        shape, _ptr(x8, "x8", (torch.uint8,), T * H), _ptr(xs, "xs", (torch.uint8,), T * H // 32),
        _ptr(offsets, "offsets", (torch.int32,)), _ptr(perm_src, "perm_src", (torch.int32,)), d13,
        _ptr(h, "h", _BF16_LIKE, rows * I), _ptr(h8, "h8", (torch.uint8,), rows * I),
        _ptr(hs, "hs", (torch.uint8,), rows * I // 32), _stream(stream)))


def moe4_expert_down_w4a8(shape: Shape, h8, hs, offsets, w2: DeviceW4, y, stream=None) -> None:
    rows = shape.T * shape.k if offsets is not None else shape.T
    d2 = w2.desc()
    check(_lib.load().moe4_expert_down_w4a8(
        shape, _ptr(h8, "h8", (torch.uint8,), rows * shape.I), _ptr(hs, "hs", (torch.uint8,), rows * shape.I // 32),
        _ptr(offsets, "offsets", (torch.int32,)), d2, _ptr(y, "y", _BF16_LIKE, rows * shape.H), _stream(stream)))


def moe4_layer_w4a8(shape: Shape, x, w_router, logits, w13: DeviceW4, w2: DeviceW4,
                    shared13: Optional[DeviceW4], shared2: Optional[DeviceW4], residual, gamma,
                    topk_idx, topk_w, residual_out, normed_out, ws, stream=None) -> None:
    """The whole layer with the FP8 (W4A8) expert FFNs."""
    T, H, E, k = shape.T, shape.H, shape.E, shape.k
    d13, d2 = w13.desc(), w2.desc()
    s13 = shared13.desc() if shared13 is not None else None
    s2 = shared2.desc() if shared2 is not None else None
    check(_lib.load().moe4_layer_w4a8(
        shape, _ptr(x, "x", _BF16_LIKE, T * H), _ptr(w_router, "w_router", _BF16_LIKE, E * H),
        _ptr(logits, "logits", (torch.float32,), T * E), d13, d2, s13, s2,
        _ptr(residual, "residual", _BF16_LIKE, T * H), _ptr(gamma, "gamma", _BF16_LIKE, H),
        _ptr(topk_idx, "topk_idx", (torch.int32,), T * k),
        _ptr(topk_w, "topk_w", (torch.float32,), T * k),
        _ptr(residual_out, "residual_out", _BF16_LIKE, T * H),
        _ptr(normed_out, "normed_out", _BF16_LIKE, T * H),
        _ptr(ws, "ws"), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


_SIDE_EVENTS = {}


def side_events():
    """Two events of the current device for moe4_layer's fork and join, created once
    (recorded once here so that they exist; make the first call outside graph capture)."""
    dev = torch.cuda.current_device()
    if dev not in _SIDE_EVENTS:
        evs = (torch.cuda.Event(), torch.cuda.Event())
        for ev in evs:
            ev.record()
        _SIDE_EVENTS[dev] = evs
    return _SIDE_EVENTS[dev]
